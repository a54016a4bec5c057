// kernels.hpp -- gfx950 kernels of the SPECTRE spectral mix.
//
// The operation (SPECTRE FFT-attention article, section 2.2 and its
// pseudocode; section 2.3 for truncation): per column (b, h, d) of length L,
// y = irfft( G[h][f] / L * Q[f] conj(K[f]) V[f] * [f < keep] ), then
// out = LayerNorm_{H*D}(x + y).  Variants: a logit gate (G = sigmoid of the
// given values, section 3.1), a complex gate (section 2.4's rotation inside
// G(f)), and the pre-norm order out = x + LayerNorm(y) (section 3.3).
//
// Data path.  Two real channels (2j, 2j+1) of one token share a complex
// number z = x[2j] + i x[2j+1] (the article's section 3.1 treats re/im as two
// real channels; here two neighbouring channels are packed the same way), so
// one complex transform of length L carries two real columns and every
// global access is a contiguous 8-byte (f32) or 4-byte (bf16) pair with lanes
// running along the contiguous H*D axis.
//
// The length factors as L = L1 * L2 * L3 (four-step / six-step
// decomposition).  With n = n1 (L2 L3) + m2 L3 + m3 and
// f = k1 + L1 (k2 + L2 k3):
//   A1  L1-point DFT over n1 per (m, pair), times w_L^{m k1}          -> T[k1][m]
//   A2  L2-point DFT over m2 per (k1, m3, pair), times w_M^{m3 k2}     (in place)
//   B   L3-point DFT over m3 per column (k1, k2), LDS-resident Stockham; the
//       spectral product for the column and its mirror column; the inverse
//       L3-point DFT over k3; times w_M^{-m3 k2} (and w_L^{-m3 k1} when
//       L2 = 1, standing in for C2's twiddle)                          -> U (in place)
//   C2  inverse L2-point DFT over k2, times w_L^{-m k1}                (in place)
//   C1  inverse L1-point DFT over k1, residual, LayerNorm              -> out
// M = L2 L3.  A pass whose size is 1 is skipped.  For L <= 2048, and for
// L = 3072 and 4096 (the single-pass column kernel k_col), the whole column
// fits one workgroup's LDS and only B runs (then a LayerNorm pass).
//
// Separating the two packed real spectra needs Z[f] and Z[L-f]; f and L-f
// always sit in a column pair {(k1, k2), (k1', k2')} (or in one self-paired
// column), which is why one B workgroup owns a column and its mirror.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dft.hpp"

namespace spectre {

enum InKind { IN_F32 = 0, IN_BF16 = 1, IN_C32 = 2 };
enum TwKind { TW_NONE = 0, TW_A1 = 1, TW_A2 = 2, TW_C2 = 3 };

// ------------------------------------------------------------- storage I/O
//
// Every tensor and spectrum is read exactly once per call, so all of them
// are loaded nontemporally: the read stream then does not push out of L2
// the lines that the row-layout stores of the LDS pass fill piece by piece
// (those pieces come from several workgroups; a line evicted half written
// costs a partial write to HBM).  Tables (twiddles, gate) use plain loads.

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float2 load_nt(const float2* p) {
  const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
  return make_float2(v.x, v.y);
}

// One channel pair at complex-element offset `off`: (ch 2j, ch 2j+1).
template <int IN>
__device__ __forceinline__ float2 load_pair(const void* base, int64_t off) {
  if constexpr (IN == IN_BF16) {
    uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(base) + off);
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
  } else {
    return load_nt(reinterpret_cast<const float2*>(base) + off);
  }
}

// Element size of one channel pair in storage kind IN, in bytes.
template <int IN>
constexpr int pair_bytes() {
  return IN == IN_BF16 ? 4 : 8;
}

// One channel pair at `ubase + off` bytes, where `ubase` is uniform across
// the wave and `off` a 32-bit per-lane offset: this is the scalar-base +
// vector-offset addressing form, so a row of R such loads costs scalar adds
// for the bases and one shared offset register.
template <int IN>
__device__ __forceinline__ float2 load_pair_u(const char* ubase, uint32_t off) {
  if constexpr (IN == IN_BF16) {
    uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ubase + off));
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
  } else {
    return load_nt(reinterpret_cast<const float2*>(ubase + off));
  }
}

// The same with a plain (cached) load: for rows whose 128-byte lines are
// shared by several workgroups, which must find them in L2.
template <int IN>
__device__ __forceinline__ float2 load_pair_c(const char* ubase, uint32_t off) {
  if constexpr (IN == IN_BF16) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(ubase + off);
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float2*>(ubase + off);
  }
}

// binary32 -> bfloat16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int OUT>
__device__ __forceinline__ void store_pair(void* base, int64_t off, float2 v) {
  if constexpr (OUT == IN_BF16) {
    uint32_t u = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
    __builtin_nontemporal_store(u, reinterpret_cast<uint32_t*>(base) + off);
  } else {
    float2* p = reinterpret_cast<float2*>(base) + off;
    __builtin_nontemporal_store(v.x, &p->x);
    __builtin_nontemporal_store(v.y, &p->y);
  }
}

__device__ __forceinline__ float2 twiddle_lookup(const float2* __restrict__ tw, int e, bool inverse) {
  float2 w = tw[e];
  return inverse ? make_float2(w.x, -w.y) : w;
}

// ------------------------------------------------------------- gate table
//
// Gate kinds (SPECTRE article: section 2.2's learnable G(f); section 3.1's
// sigmoid gate; section 2.4's relative position as a frequency-dependent
// rotation inside G(f)):
//   GATE_REAL    gate [H][nbins]: the multiplier itself;
//   GATE_LOGIT   gate [H][nbins]: logits, multiplier 1 / (1 + exp(-G));
//   GATE_COMPLEX gate [H][nbins][2]: real and imaginary parts.
// The multiplier of full-spectrum bin f (0 <= f < L) is the gate of bin
// fc = min(f, L - f), conjugated for f > L/2 (the Hermitian extension of the
// product); at f = 0 and f = L/2 only its real part acts, as the inverse
// real transform reads only the real part of those bins.

enum GateKind { GATE_REAL = 0, GATE_LOGIT = 1, GATE_COMPLEX = 2 };

// scale * multiplier of full-spectrum bin f of head h (fc = min(f, L - f) < keep).
__device__ __forceinline__ float2 gate_value(const float* gate, int kind, int64_t nbins, int64_t h,
                                             int64_t fc, int64_t f, int64_t L, float scale) {
  if (kind == GATE_COMPLEX) {
    const float2 g = reinterpret_cast<const float2*>(gate)[h * nbins + fc];
    const bool real_bin = f == 0 || 2 * f == L;
    return make_float2(g.x * scale, real_bin ? 0.f : (2 * f > L ? -g.y : g.y) * scale);
  }
  float a = gate[h * nbins + fc];
  if (kind == GATE_LOGIT) a = 1.0f / (1.0f + expf(-a));
  return make_float2(a * scale, 0.f);
}

// gtab[(h * ncol + c) * N + k3] = scale * the multiplier of bin f if that bin
// is kept, else 0, for column c = kc + L1 * k2c and f = kc + L1 * (k2c + L2 *
// k3): the gate of every bin in the order the square B kernel's lanes visit
// them, so that 32 lanes of one column read 32 consecutive values (binary32
// values, or binary32 pairs for a complex gate).  Built by an extra grid
// plane of the first strided pass (multi-level plans only: a single-level
// square kernel reads the gate itself).

struct GateTabParams {
  const float* gate;  // [H][nbins], or [H][nbins][2] for a complex gate
  float* gtab;        // [H][ncol][N] (pairs for a complex gate); null: no table to build
  int64_t L;
  int L1, L2, N, ncol, nbins;
  int64_t keep, total;  // total = H * L
  float scale;
  int kind;  // GateKind
};

// Entries idx0, idx0 + stride, ... of the table.
__device__ __forceinline__ void gate_table_fill(const GateTabParams& p, int64_t idx0, int64_t stride) {
  for (int64_t idx = idx0; idx < p.total; idx += stride) {
    const int k3 = (int)(idx % p.N);
    const int64_t r = idx / p.N;
    const int c = (int)(r % p.ncol);
    const int h = (int)(r / p.ncol);
    const int64_t f = c % p.L1 + (int64_t)p.L1 * (c / p.L1 + (int64_t)p.L2 * k3);
    const int64_t fc = f < p.L - f ? f : p.L - f;
    const float2 g = fc < p.keep ? gate_value(p.gate, p.kind, p.nbins, h, fc, f, p.L, p.scale)
                                 : make_float2(0.f, 0.f);
    if (p.kind == GATE_COMPLEX)
      reinterpret_cast<float2*>(p.gtab)[idx] = g;
    else
      p.gtab[idx] = g.x;
  }
}

// ------------------------------------------------------ strided DFT passes
//
// Data viewed as [outer][R][inner][CP2] complex elements (CP2 = H*D/2 channel
// pairs).  Each thread owns one (outer, inner, pair) line: R loads along the
// middle axis, an R-point DFT in registers, a twiddle per output, R stores to
// the same positions.  Lanes run along the pair axis, so every load/store
// instruction of a wave touches 64 consecutive pairs.
//
// blockIdx.y selects the tensor (q, k, v) for the forward passes (and, for
// the split kernel, 3 the gate table).

struct StridedParams {
  const void* in[3];
  float2* out[3];
  const float2* twL;  // twL[e] = exp(-2 pi i e / L)
  int64_t outer, inner, CP2;
  int L1;
  GateTabParams gt;   // k_strided_split: blockIdx.y == 3 builds this table
};

// TILED (the forward first pass of a two-level plan, or the second pass of
// a three-level one, out of place): the outputs of row block r go to
// [outer][r][CP2 / 4][inner][4] like the tiled split pass; a wave covers
// 4 rows x 16 pairs and a workgroup 16 rows x 16 pairs, so reads come in
// 64- or 128-byte row pieces and each 4-pair block gets 16 rows = 512
// contiguous bytes from the workgroup.  Needs inner % 16 == 0 and
// CP2 % 16 == 0.  blockIdx.y == 3, when launched, builds the gate table.
template <int R, int IN, int TW, int SIGN, bool TILED = false>
__global__ __launch_bounds__(256) void k_strided(StridedParams p) {
  if (blockIdx.y == 3) {  // the gate table, folded into this launch
    gate_table_fill(p.gt, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                    (int64_t)gridDim.x * blockDim.x);
    return;
  }
  int64_t cp, o, cp0 = 0;
  int i, i0 = 0;
  if constexpr (TILED) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t pgs = p.CP2 / 16, tiles = (p.inner / 16) * pgs;
    const int64_t g = blockIdx.x;
    o = g / tiles;
    if (o >= p.outer) return;
    const int64_t rem = g - o * tiles;
    i0 = (int)(rem / pgs) * 16;
    cp0 = (rem % pgs) * 16;
    i = i0 + 4 * w + (lane >> 4);
    cp = cp0 + (lane & 15);
  } else {
    const int64_t line = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t lines = p.outer * p.inner * p.CP2;
    if (line >= lines) return;
    cp = line % p.CP2;
    const int64_t t = line / p.CP2;
    i = (int)(t % p.inner);
    o = t / p.inner;
  }
  const void* in = p.in[blockIdx.y];
  float2* out = p.out[blockIdx.y];
  const int64_t step = p.inner * p.CP2;
  const int64_t base = (o * R * p.inner + i) * p.CP2 + cp;
  const int64_t obase = TILED ? o * R * step + (cp >> 2) * (p.inner * 4) + i * 4 + (cp & 3) : base;

  float2 a[R];
#pragma unroll
  for (int r = 0; r < R; ++r) a[r] = load_pair<IN>(in, base + r * step);
  dft<R, SIGN>(a);
  auto twiddled = [&](int r) __attribute__((always_inline)) {
    float2 v = a[r];
    if constexpr (TW == TW_A1) {
      if (r != 0 && i != 0) v = cmul(v, twiddle_lookup(p.twL, i * r, false));
    } else if constexpr (TW == TW_A2) {
      if (r != 0 && i != 0) v = cmul(v, twiddle_lookup(p.twL, i * r * p.L1, false));
    } else if constexpr (TW == TW_C2) {
      const int k1 = (int)(o % p.L1);
      const int e = (r * (int)p.inner + i) * k1;
      if (e != 0) v = cmul(v, twiddle_lookup(p.twL, e, true));
    }
    return v;
  };
  if constexpr (TILED) {
    // the workgroup's 16 rows x 16 pairs of each output row block are 4
    // blocks of 16 rows x 4 pairs = 512 contiguous bytes; outputs go through
    // LDS 8 at a time so that every store instruction writes a whole block
    __shared__ float2 stg[8][16][17];
    const int tid = threadIdx.x;
    const int rl = tid >> 4, pl = tid & 15;  // = 4 w + lane / 16, lane % 16
    float2* ob = out + o * R * step + (cp0 >> 2) * (p.inner * 4) + i0 * 4;
#pragma unroll
    for (int r0 = 0; r0 < R; r0 += 8) {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr)
        if (r0 + rr < R) stg[rr][rl][pl] = twiddled(r0 + rr);
      __syncthreads();
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        // element e = e2 * 256 + tid: pair pr, row r, block blk, local output rr
        const int e = e2 * 256 + tid;
        const int pr = e & 3, r = (e >> 2) & 15, blk = (e >> 6) & 3, rr = e >> 8;
        if (r0 + rr < R) ob[(int64_t)(r0 + rr) * step + blk * (p.inner * 4) + r * 4 + pr] = stg[rr][r][4 * blk + pr];
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) out[obase + r * step] = twiddled(r);
  }
}

// Radix-2 join of an R-point DFT split over lanes l (h = 0, the even
// samples) and l^32 (h = 1, the odd samples), each holding its R/2-point DFT
// in v[0 .. R/2).  One v_permlane32_swap per dword pairs v[n] of the low
// half with v[n + Q] of the high half (Q = R/4): lane h then holds E0 and E1
// at index n + Q h and finishes the butterfly in place, so v[n] becomes
// output n + Q h and v[n + Q] output n + Q h + R/2.  The twiddle
// w^(n + Q h), w = exp(SIGN 2 pi i / R), is w^n times w^Q = SIGN i on h = 1.
template <int R, int SIGN>
__device__ __forceinline__ void join_swap(float2 (&v)[R / 2], int h) {
  constexpr int Q = R / 4;
  static_assert(R % 4 == 0, "join_swap needs R divisible by 4");
#pragma unroll
  for (int n = 0; n < Q; ++n) {
    const auto sx = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[n].x), __float_as_uint(v[n + Q].x),
                                                     false, false);
    const auto sy = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[n].y), __float_as_uint(v[n + Q].y),
                                                     false, false);
    const float2 e0 = make_float2(__uint_as_float(sx[0]), __uint_as_float(sy[0]));
    float2 t = twiddle_ct<R, SIGN>(make_float2(__uint_as_float(sx[1]), __uint_as_float(sy[1])), n);
    if (h) t = SIGN > 0 ? make_float2(-t.y, t.x) : make_float2(t.y, -t.x);
    v[n] = cadd(e0, t);
    v[n + Q] = csub(e0, t);
  }
}

// Forward strided pass with the R-point DFT split over two lanes (l, l^32):
// lane half h loads the samples r = 2a + h (a < R/2) and transforms them
// (R/2 points); the halves trade results with a lane permute and finish
// with a radix-2 step, X[k] = E0[k] + w_R^k E1[k] on half 0 and
// X[k + R/2] = E0[k] - w_R^k E1[k] on half 1.  Half the registers of the
// one-lane form, so more waves hide the memory latency.  A wave covers 32
// lines; both lanes of a line are active or neither is.
//
// Row output (TILED = false): a wave's 32 lines are 32 consecutive pairs of
// one row, written back to the same positions ([outer][R][inner][CP2]).
// Tiled output (TILED = true, used for the first pass of a two-level plan):
// the outputs of row block r go to [outer][r][CP2 / 4][inner][4], so that
// the LDS pass finds the inner rows of 4 channel pairs contiguous.  A wave
// covers RW rows x 32 / RW pairs and a workgroup 4 RW consecutive rows:
// binary32 inputs use RW = 2 (reads: 128-byte row pieces; writes: 8 rows x
// 4 pairs = 256 contiguous bytes per block over the 4 waves), bfloat16
// inputs RW = 1 (reads: 32 pairs = 128 bytes of one row; writes: 4 rows x
// 4 pairs = 128 bytes per block).  Needs inner % 8 == 0 and CP2 % 32 == 0.
template <int R, int IN, int TW, bool TILED>
__global__ __launch_bounds__(256) void k_strided_split(StridedParams p) {
  if (blockIdx.y == 3) {  // the gate table, folded into this launch
    gate_table_fill(p.gt, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                    (int64_t)gridDim.x * blockDim.x);
    return;
  }
  constexpr int R2 = R / 2;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int64_t gw = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;  // global wave
  int64_t cp, o, cp0 = 0;
  int i, i0 = 0;
  if constexpr (TILED) {
    constexpr int RW = IN == IN_BF16 ? 1 : 2;  // rows per wave
    constexpr int PW = 32 / RW;                // pairs per wave
    const int c = lane & 31;
    const int64_t g = gw >> 2;
    const int64_t pgs = p.CP2 / PW, tiles = (p.inner / (4 * RW)) * pgs;
    o = g / tiles;
    if (o >= p.outer) return;
    const int64_t rem = g - o * tiles;
    i0 = (int)(rem / pgs) * (4 * RW);
    cp0 = (rem % pgs) * PW;
    i = i0 + RW * (int)(gw & 3) + c / PW;
    cp = cp0 + c % PW;
  } else {
    const int64_t line = gw * 32 + (lane & 31);
    const int64_t lines = p.outer * p.inner * p.CP2;
    if (line >= lines) return;
    cp = line % p.CP2;
    const int64_t t = line / p.CP2;
    i = (int)(t % p.inner);
    o = t / p.inner;
  }
  const int64_t step = p.inner * p.CP2;  // pairs between rows r and r + 1
  const int64_t base = (o * R * p.inner + i) * p.CP2 + cp;
  const char* in = reinterpret_cast<const char*>(p.in[blockIdx.y]) + (base + h * step) * pair_bytes<IN>();
  const int64_t obase = TILED ? o * R * step + (cp >> 2) * (p.inner * 4) + i * 4 + (cp & 3) : base;
  char* out = reinterpret_cast<char*>(p.out[blockIdx.y]) + (obase + h * R2 * step) * 8;

  float2 e[R2];
#pragma unroll
  for (int a = 0; a < R2; ++a) {
    e[a] = load_pair_u<IN>(in, (uint32_t)0);
    in += 2 * step * pair_bytes<IN>();
  }
  // twiddle w^k1 for output k1 = k + R2 h, w = w_L^i (A1) or w_L^(i L1) (A2):
  // seeds w^(R2 h + j), j < 4, times (w^4)^(k / 4), 5 table loads per lane.
  const int tw_i = TW == TW_A2 ? i * p.L1 : i;
  dft<R2, -1>(e);
  float2 tws[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tws[j] = p.twL[tw_i * (R2 * h + j)];
  const float2 tw4 = p.twL[4 * tw_i];
  float2 stp = make_float2(1.f, 0.f);
  auto output = [&](int k) __attribute__((always_inline)) {
    const float2 mine = e[k];
    // the partner lane l ^ 32's value: one v_permlane32_swap per dword (VALU,
    // no LDS round trip; 1.5 us faster than a bpermute at 65536 tokens)
    const auto sx = __builtin_amdgcn_permlane32_swap(__float_as_uint(mine.x), __float_as_uint(mine.x), false, false);
    const auto sy = __builtin_amdgcn_permlane32_swap(__float_as_uint(mine.y), __float_as_uint(mine.y), false, false);
    const float2 other = h ? make_float2(__uint_as_float(sx[0]), __uint_as_float(sy[0]))
                           : make_float2(__uint_as_float(sx[1]), __uint_as_float(sy[1]));
    const float2 e0 = h ? other : mine;
    const float2 e1 = twiddle_ct<R, -1>(h ? mine : other, k);
    float2 xk = h ? csub(e0, e1) : cadd(e0, e1);
    xk = cmul(xk, cmul(tws[k & 3], stp));
    if ((k & 3) == 3) stp = cmul(stp, tw4);
    return xk;
  };
  if constexpr (TILED) {
    // The workgroup covers RWG = 4 RW rows x PWG = 32 / RW pairs; each output
    // row block holds PWG / 4 blocks of RWG rows x 4 pairs (128 or 256
    // contiguous bytes).  Outputs go through LDS KB k at a time (2 KB row
    // blocks with both halves) so that each store instruction writes whole
    // blocks: 16 for binary32 inputs (two rounds of 32-point halves, 35 KB of
    // LDS, fewer barriers: measured 2.5 us faster at 65536 tokens), 8 for
    // bfloat16 (where 16 measured slower).
    constexpr int RW = IN == IN_BF16 ? 1 : 2, RWG = 4 * RW, PWG = 32 / RW;
    constexpr int KB = IN != IN_BF16 && R2 % 16 == 0 ? 16 : 8;
    __shared__ float2 stg[2 * KB][RWG][PWG + 1];
    const int rl = RW * (int)(gw & 3) + (lane & 31) / PWG, pl = (lane & 31) % PWG;
    const int tid = threadIdx.x;
    char* obase_wg = reinterpret_cast<char*>(p.out[blockIdx.y]) +
                     (o * R * step + (cp0 >> 2) * (p.inner * 4) + i0 * 4) * 8;
#pragma unroll
    for (int k0 = 0; k0 < R2; k0 += KB) {
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) stg[kk + KB * h][rl][pl] = output(k0 + kk);
      __syncthreads();
#pragma unroll
      for (int e2 = 0; e2 < KB; ++e2) {
        // element e = e2 * 256 + tid: pair pr, row r, block blk, local row block kl
        const int e = e2 * 256 + tid;
        const int pr = e & 3, r = (e >> 2) % RWG, blk = ((e >> 2) / RWG) % (PWG / 4), kl = e >> 7;
        const int k1 = k0 + (kl % KB) + R2 * (kl / KB);
        *reinterpret_cast<float2*>(obase_wg + ((int64_t)k1 * step + blk * (p.inner * 4) + r * 4 + pr) * 8) =
            stg[kl][r][4 * blk + pr];
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int k = 0; k < R2; ++k) *reinterpret_cast<float2*>(out + (int64_t)k * step * 8) = output(k);
  }
}

// ------------------------------------------- B: LDS Stockham + spectral mix

struct MidParams {
  const void* in[3];     // q, k, v sources (raw tensors, or the A-pass output)
  float2* out;           // inverse output (may alias in[0])
  const float* gate;     // [H][nbins]
  const float* gtab;     // k_mid_sq: [H][ncol][N] gate table (scale, truncation, mirror folded
                         // in), or null for a single-level plan, which reads gate directly
  int gate_kind;         // GateKind of gate (gtab: binary32 pairs for a complex gate)
  int ncol;              // columns per batch element, L1 * L2
  int tiled;             // k_mid_sq: in[] laid out [b][column][CP2 / 4][N][4] (see k_strided_split)
  const float2* twN;     // twN[e] = exp(-2 pi i e / N), e < N
  const float2* twL;     // twL[e] = exp(-2 pi i e / L)
  const int2* wgcols;    // per workgroup: its column(s), col = k1 + L1 * k2 (-1 = none)
  int L, L1, L2, N, M, CP2, D, keep, nbins;
  int nslot, cpt, Tc;
  int selfwg;            // workgroup index holding the two self-paired columns, or -1
  int nrad;
  int rad[8];            // Stockham radices, product N
  float scale;           // 1 / (8 L^2): the mix's 1/L, the inverse's 1/L, the (1/2)^3 of the split
  int gx, gy, gz;        // k_mid_dma: the work items (column pairs, channel-pair blocks, batch)
  // chunked mix: bin 0 of column (0, 0) -- the column sums of each block --
  // times dc_scale = 1 / L goes to dc[x * dc_stride + b * CP2 + pair] (the
  // block means of q, k, v); null otherwise
  float2* dc;
  int64_t dc_stride;
  float dc_scale;
};

// One Stockham autosort pass of radix R over the LDS-resident columns.
// Thread (tc, col) owns butterflies j = tc + Tc*b, b < P/R; butterfly j reads
// x[j + r N/R], applies exp(sign 2 pi i r (j mod Ns) / (Ns R)), does an R-point
// DFT and writes x[(j / Ns) Ns R + (j mod Ns) + r Ns].  The first pass reads
// and the last pass writes the thread's registers directly: there the data
// sits at x[tc + Tc i] = v[i].
template <int P, int R, int SIGN>
__device__ __forceinline__ void stockham_pass(float2 (&v)[P], float2* lds, int N, int Ns, int Tc,
                                              int tc, int col, int ncols, const float2* __restrict__ twN,
                                              bool first, bool last) {
  if constexpr (P % R != 0) {
    return;  // never planned: the host only picks radices that divide P
  } else {
    constexpr int NB = P / R;
    float2 u[NB][R];
    const int NR = N / R;
    if (first) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < R; ++r) u[b][r] = v[b + r * NB];
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int j = tc + Tc * b;
#pragma unroll
        for (int r = 0; r < R; ++r) u[b][r] = lds[(j + r * NR) * ncols + col];
      }
      __syncthreads();
    }
    const int tstride = N / (Ns * R);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = tc + Tc * b;
      const int k = j % Ns;
      if (Ns > 1) {
#pragma unroll
        for (int r = 1; r < R; ++r) u[b][r] = cmul(u[b][r], twiddle_lookup(twN, r * k * tstride, SIGN > 0));
      }
      dft<R, SIGN>(u[b]);
      if (last) {
#pragma unroll
        for (int r = 0; r < R; ++r) v[b + r * NB] = u[b][r];
      } else {
        const int base = (j / Ns) * Ns * R + k;
#pragma unroll
        for (int r = 0; r < R; ++r) lds[(base + r * Ns) * ncols + col] = u[b][r];
      }
    }
    if (!last) __syncthreads();
  }
}

// Full N-point transform of every column; in and out: v[i] = x[tc + Tc i].
// The LDS buffer must be free on entry (caller synchronises).
template <int P, int SIGN>
__device__ __forceinline__ void fft_columns(float2 (&v)[P], float2* lds, const MidParams& p, int tc, int col,
                                            int ncols) {
  int Ns = 1;
  for (int s = 0; s < p.nrad; ++s) {
    const int R = p.rad[s];
    const bool first = s == 0, last = s == p.nrad - 1;
    switch (R) {
      case 2: stockham_pass<P, 2, SIGN>(v, lds, p.N, Ns, p.Tc, tc, col, ncols, p.twN, first, last); break;
      case 3: stockham_pass<P, 3, SIGN>(v, lds, p.N, Ns, p.Tc, tc, col, ncols, p.twN, first, last); break;
      case 4: stockham_pass<P, 4, SIGN>(v, lds, p.N, Ns, p.Tc, tc, col, ncols, p.twN, first, last); break;
      case 6: stockham_pass<P, 6, SIGN>(v, lds, p.N, Ns, p.Tc, tc, col, ncols, p.twN, first, last); break;
      case 8: stockham_pass<P, 8, SIGN>(v, lds, p.N, Ns, p.Tc, tc, col, ncols, p.twN, first, last); break;
      case 12: stockham_pass<P, 12, SIGN>(v, lds, p.N, Ns, p.Tc, tc, col, ncols, p.twN, first, last); break;
      case 16: stockham_pass<P, 16, SIGN>(v, lds, p.N, Ns, p.Tc, tc, col, ncols, p.twN, first, last); break;
      default: break;
    }
    Ns *= R;
  }
}

// The i-th frequency pair a thread owns in the spectral product: element e
// (slot se, index ie) and its mirror e' (the bin L - f of e's bin f).
struct PairRef {
  int se, ie, sm, im;
};

__device__ __forceinline__ bool pair_at(int i, int P, int s, int tc, int Tc, int N, bool regular,
                                        PairRef& pr) {
  if (regular) {
    // slot 0 holds column c, slot 1 its mirror column: bin (0, idx) <-> (1, N-1-idx)
    if (i >= P / 2) return false;
    pr.se = 0;
    pr.ie = tc + Tc * (2 * i + s);
    pr.sm = 1;
    pr.im = N - 1 - pr.ie;
    return true;
  }
  // self-paired column in slot s: index idx <-> (a - idx) mod N with a = 0
  // for column (0, 0) (slot 0) and a = N - 1 for the other one (slot 1)
  const bool a_zero = s == 0;
  pr.se = pr.sm = s;
  if (i < P / 2) {
    pr.ie = tc + Tc * i;
    pr.im = a_zero ? (N - pr.ie) % N : N - 1 - pr.ie;
    return true;
  }
  if (i == P / 2 && a_zero && tc == 0) {
    pr.ie = pr.im = N / 2;
    return true;
  }
  return false;
}

// Work-group ids go to the 8 XCDs round-robin (id mod 8), each XCD with its
// own L2.  Renumbered so that XCD x runs a contiguous eighth of the grid in
// its natural order, the work-groups that share cache lines (neighbouring
// channel-pair blocks of one column) share an L2 and run close in time.  A
// tail beyond a multiple of 8 keeps its own ids.
__device__ __forceinline__ int3 xcd_grouped_block() {
  const unsigned gx = gridDim.x, gy = gridDim.y;
  const unsigned total = gx * gy * gridDim.z;
  unsigned lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const unsigned per = total / 8;
  if (lin < per * 8) lin = (lin % 8) * per + lin / 8;
  return make_int3((int)(lin % gx), (int)((lin / gx) % gy), (int)(lin / (gx * gy)));
}

// Block order for the multi-level square B pass, whose workgroup writes 32
// bytes (4 channel pairs) of each output row: the 4 workgroups that fill
// one 128-byte line (channel-pair blocks 4 q .. 4 q + 3 of one column pair)
// get ids 8 apart, so they run on one XCD one after another and the line is
// whole before L2 evicts it.  Groups of 4 go to the XCDs round-robin.
// Needs gridDim.y % 4 == 0 and a grid size that is a multiple of 32;
// otherwise the natural order.
__device__ __forceinline__ int3 sharer_block_of(unsigned lin, unsigned gx, unsigned gy, unsigned gz) {
  const unsigned total = gx * gy * gz;
  if (gy % 4 != 0 || total % 32 != 0)
    return make_int3((int)(lin % gx), (int)((lin / gx) % gy), (int)(lin / (gx * gy)));
  const unsigned w = (lin / 8) % 4;             // position in the group
  const unsigned g = lin % 8 + 8 * (lin / 32);  // group: one column pair, 4 channel-pair blocks
  const unsigned rest = g / gx, yq = gy / 4;
  return make_int3((int)(g % gx), (int)(4 * (rest % yq) + w), (int)(rest / yq));
}

__device__ __forceinline__ int3 sharer_grouped_block() {
  return sharer_block_of(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), gridDim.x,
                         gridDim.y, gridDim.z);
}

template <int P, int IN>
__global__ __launch_bounds__(512) void k_mid(MidParams p) {
  extern __shared__ float2 lds[];
  const int3 blk = xcd_grouped_block();
  const int ncols = p.nslot * p.cpt;
  const int tid = threadIdx.x;
  const int col = tid % ncols;
  const int tc = tid / ncols;
  const int s = col / p.cpt;
  const int j = col - s * p.cpt;
  const int cp = blk.y * p.cpt + j;
  const int b = blk.z;
  const int2 cols = p.wgcols[blk.x];
  const int my_col = s == 0 ? cols.x : cols.y;
  const bool regular = p.nslot == 2 && blk.x != p.selfwg;
  const bool active = my_col >= 0;
  const int k1 = active ? my_col % p.L1 : 0;
  const int k2 = active ? my_col / p.L1 : 0;
  const int64_t gbase = (((int64_t)b * p.L1 + k1) * p.M + (int64_t)k2 * p.N) * p.CP2 + cp;

  constexpr int NPR = P / 2 + 1;
  float2 v[P];
  float2 sa[NPR], sb[NPR];

#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const void* src = p.in[x];
    if (active) {
#pragma unroll
      for (int i = 0; i < P; ++i) v[i] = load_pair<IN>(src, gbase + (int64_t)(tc + p.Tc * i) * p.CP2);
    } else {
#pragma unroll
      for (int i = 0; i < P; ++i) v[i] = make_float2(0.f, 0.f);
    }
    __syncthreads();  // LDS free: the previous tensor's product step is done
    fft_columns<P, -1>(v, lds, p, tc, col, ncols);
    if (p.dc != nullptr && my_col == 0 && tc == 0)  // bin 0 of column (0, 0)
      p.dc[x * p.dc_stride + (int64_t)b * p.CP2 + cp] = cscale(v[0], p.dc_scale);
#pragma unroll
    for (int i = 0; i < P; ++i) lds[(tc + p.Tc * i) * ncols + col] = v[i];
    __syncthreads();

    // split the two packed real spectra and accumulate the product:
    // 2A = Z[f] + conj Z[L-f], 2B = -i (Z[f] - conj Z[L-f])
#pragma unroll
    for (int i = 0; i < NPR; ++i) {
      PairRef pr;
      if (!pair_at(i, P, s, tc, p.Tc, p.N, regular, pr)) continue;
      const int oe = pr.ie * ncols + pr.se * p.cpt + j;
      const int om = pr.im * ncols + pr.sm * p.cpt + j;
      const float2 z = lds[oe], zm = lds[om];
      const float2 A = make_float2(z.x + zm.x, z.y - zm.y);
      const float2 Bv = make_float2(z.y + zm.y, zm.x - z.x);
      if (x == 0) {
        sa[i] = A;
        sb[i] = Bv;
      } else if (x == 1) {
        sa[i] = cmulc(sa[i], A);
        sb[i] = cmulc(sb[i], Bv);
      } else {
        // bin of element e and the gate of each packed channel's head
        const int se_col = pr.se == 0 ? cols.x : cols.y;
        const int f = se_col % p.L1 + p.L1 * (se_col / p.L1 + p.L2 * pr.ie);
        const int fc = min(f, p.L - f);
        float2 ga = make_float2(0.f, 0.f), gb = ga;
        if (fc < p.keep) {
          ga = gate_value(p.gate, p.gate_kind, p.nbins, (2 * cp) / p.D, fc, f, p.L, p.scale);
          gb = gate_value(p.gate, p.gate_kind, p.nbins, (2 * cp + 1) / p.D, fc, f, p.L, p.scale);
        }
        const float2 oa = cmul(cmul(sa[i], A), ga);
        const float2 ob = cmul(cmul(sb[i], Bv), gb);
        // W[f] = Oa + i Ob, W[L-f] = conj(Oa) + i conj(Ob)
        lds[oe] = make_float2(oa.x - ob.y, oa.y + ob.x);
        lds[om] = make_float2(oa.x + ob.y, ob.x - oa.y);
      }
    }
  }
  __syncthreads();

  // inverse transform of W along k3, then the twiddle w_M^{-m3 k2}; when there
  // is no L2 pass (L2 = 1, m = m3) the twiddle w_L^{-m k1} of the inverse
  // four-step joins it here
#pragma unroll
  for (int i = 0; i < P; ++i) v[i] = lds[(tc + p.Tc * i) * ncols + col];
  __syncthreads();
  fft_columns<P, +1>(v, lds, p, tc, col, ncols);
  if (!active) return;
  const int tw_mul = p.L1 * k2 + (p.L2 == 1 ? k1 : 0);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int m3 = tc + p.Tc * i;
    float2 w = v[i];
    if (tw_mul != 0 && m3 != 0) w = cmul(w, twiddle_lookup(p.twL, m3 * tw_mul, true));
    p.out[gbase + (int64_t)m3 * p.CP2] = w;
  }
}

// -------------------------------- B for N = R * R: two register DFTs
//
// The same pass as k_mid, specialised for column length N = R^2 (R = 16 or
// 32).  Each transform is an R-point DFT in registers, one padded LDS
// transpose, and a second R-point DFT in registers (the four-step split of
// N itself), so a transform costs one LDS round trip and every index is a
// compile-time constant.
//
//   stage 1 (coalesced mapping: thread (t, col), column fastest):
//     v[k] = sum_i x[t + R i] w_R^{ik} * w_N^{t k}          -> LDS [k][t][col]
//   stage 2 (mirror mapping: R lanes per column, the two columns of a pair
//   in one wave): thread k1 reads [k1][t][col] and gets X[k1 + R k2], k2 < R.
//
// The mirror bin of (k1, k2) is held by a lane of the same wave: for a
// column and its mirror column it is lane (other slot, R-1-k1) at k2' = R-1-k2;
// inside column (0, 0) it is lane (R - k1) mod R (k2' = R-1-k2, or (R-k2) mod R
// when k1 = 0); inside the other self-paired column lane R-1-k1.  Each lane
// pulls its partner's upper half (k2 >= R/2) with ds_bpermute and owns the
// R/2 pairs whose own element has k2 < R/2 (lane k1 = 0 of column (0, 0)
// owns its pairs alone, plus the self-mirrored bin k2 = R/2).
//
// The inverse runs the split backwards: stage-2 lanes transform along k2,
// twiddle w_N^{-k1 n}, LDS transpose, stage-1 lanes transform along k1 and
// hold z[t + R i] -- the input distribution -- for coalesced stores.
//
// GL (multi-level plans whose workgroup's channel pairs share one head): the
// workgroup's gate values, nslot x (R/2 + 1) x R of the table, are copied to
// LDS during the first tensor, so the product reads them from LDS instead of
// waiting on global loads.

__device__ __forceinline__ float lane_pull(float v, int src_byte) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_byte, __float_as_int(v)));
}
__device__ __forceinline__ float2 lane_pull2(float2 v, int src_byte) {
  return make_float2(lane_pull(v.x, src_byte), lane_pull(v.y, src_byte));
}

template <int R, int IN, bool GL = false, bool CG = false>
__global__ __launch_bounds__(256, 2) void k_mid_sq(MidParams p) {
  constexpr int N = R * R;
  constexpr int H2 = R / 2;
  extern __shared__ float2 lds[];
  const int3 blk = p.nslot == 1 ? xcd_grouped_block()
                  : p.cpt == 4  ? sharer_grouped_block()
                                : make_int3((int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z);
  const int ncols = p.nslot * p.cpt;
  const int ROW = R * ncols + 1;  // padded: stage-2 lanes stride ROW, an odd count
  float2* twl = lds + R * ROW;     // the N-point twiddles, copied from p.twN
  float* gl = reinterpret_cast<float*>(twl + N);  // GL: gate values [slot][u <= R/2][k1]
  const int tid = threadIdx.x;

  // stage-1 / stage-3 identity
  const int col1 = tid % ncols;
  const int t1 = tid / ncols;
  const int s1 = col1 / p.cpt;
  const int j1 = col1 - s1 * p.cpt;
  // stage-2 identity
  const int G = p.nslot * R;
  const int j2 = tid / G;
  const int r2 = tid - j2 * G;
  const int s2 = r2 / R;
  const int k1 = r2 - s2 * R;
  const int col2 = s2 * p.cpt + j2;

  const int2 cols = p.wgcols[blk.x];
  const bool regular = p.nslot == 2 && blk.x != p.selfwg;
  int ps, pk1;
  bool a_zero = false;
  if (regular) {
    ps = 1 - s2;
    pk1 = R - 1 - k1;
  } else {
    ps = s2;
    a_zero = s2 == 0;
    pk1 = a_zero ? (R - k1) % R : R - 1 - k1;
  }
  const int partner_byte = (((j2 * G + ps * R + pk1) & 63) << 2);
  const bool special = a_zero && k1 == 0;

  const int b = blk.z;
  const int colid1 = s1 == 0 ? cols.x : cols.y;
  const int colid2 = s2 == 0 ? cols.x : cols.y;
  const bool active1 = colid1 >= 0;
  const int kc1 = active1 ? colid1 % p.L1 : 0, k2c1 = active1 ? colid1 / p.L1 : 0;
  const int cp1 = blk.y * p.cpt + j1;
  const int cp2 = blk.y * p.cpt + j2;
  // element i of this stage-1 lane's column sits at pair index
  //   b * L * CP2 + lane_pair + i * R * CP2
  const uint32_t lane_pair = (uint32_t)((kc1 * p.M + k2c1 * N + t1) * p.CP2 + cp1);
  const int64_t batch_pair = (int64_t)b * p.L * p.CP2;
  const int64_t row_pair = (int64_t)R * p.CP2;
  // the same element in the tiled input layout: block cp1 / 4 of the column
  // holds its N rows of 4 pairs contiguously
  const uint32_t in_pair = p.tiled ? (uint32_t)((kc1 * p.M + k2c1 * N) * p.CP2 + (cp1 >> 2) * (N * 4) +
                                                t1 * 4 + (cp1 & 3))
                                   : lane_pair;
  const int64_t in_row = p.tiled ? (int64_t)R * 4 : row_pair;
  // element (k1, k2) of the stage-2 column is bin k3 = k1 + R k2 of column colid2
  const int colid2c = colid2 >= 0 ? colid2 : 0;
  const int ha = (2 * cp2) / p.D, hb = (2 * cp2 + 1) / p.D;

  float2 v[R];
  float2 sa[H2 + 1], sb[H2 + 1];

#pragma unroll 1
  for (int x = 0; x < 3; ++x) {
    // values only one phase needs are made opaque per iteration, so they are
    // not hoisted out of the loop and kept live across it
    // gate values of this lane's bins (k1 + R u of column colid2)
    const float* gta = p.gtab + ((int64_t)ha * p.ncol + colid2c) * N + k1;
    const float* gtb = p.gtab + ((int64_t)hb * p.ncol + colid2c) * N + k1;
    int t1o = t1;  // opaque: the 31 twiddle addresses are recomputed per tensor
    asm volatile("" : "+v"(gta), "+v"(gtb), "+v"(t1o));
    // ---- stage 1: DFT over i of x[t + R i], twiddle w_N^{t k}
    {
      const char* src = reinterpret_cast<const char*>(p.in[x]) + batch_pair * pair_bytes<IN>();
      const uint32_t off = in_pair * pair_bytes<IN>();
      if (active1) {
#pragma unroll
        for (int i = 0; i < R; ++i) v[i] = load_pair_u<IN>(src + i * in_row * pair_bytes<IN>(), off);
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) v[i] = make_float2(0.f, 0.f);
      }
    }
    if (x == 0) {
      for (int e = tid; e < N; e += R * ncols) twl[e] = p.twN[e];
      if constexpr (GL) {
        const int hw = (2 * blk.y * p.cpt) / p.D;  // the workgroup's head
        for (int e = tid; e < p.nslot * (H2 + 1) * R; e += R * ncols) {
          const int sl = e / ((H2 + 1) * R), u = (e / R) % (H2 + 1), kk = e % R;
          const int c = sl == 0 ? cols.x : cols.y;
          gl[e] = p.gtab[((int64_t)hw * p.ncol + (c >= 0 ? c : 0)) * N + kk + R * u];
        }
      }
      __syncthreads();
    }
    dft<R, -1>(v);
#pragma unroll
    for (int k = 1; k < R; ++k) v[k] = cmul(v[k], twl[t1o * k]);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < R; ++k) lds[k * ROW + t1 * ncols + col1] = v[k];
    __syncthreads();
    // ---- stage 2: DFT over t -> X[k1 + R k2]
#pragma unroll
    for (int t = 0; t < R; ++t) v[t] = lds[k1 * ROW + t * ncols + col2];
    dft<R, -1>(v);
    if (p.dc != nullptr && special)  // bin 0 of column (0, 0)
      p.dc[x * p.dc_stride + (int64_t)b * p.CP2 + cp2] = cscale(v[0], p.dc_scale);

    // ---- split the packed spectra and accumulate / finish the product.
    // The mirror bin of this lane's k2 = u < R/2 is the partner lane's
    // k2 = R-1-u (pulled with ds_bpermute); lane k1 = 0 of column (0, 0)
    // holds its own mirrors at (R-u) mod R and the self-mirrored bin R/2.
    // 2A = Z[f] + conj Z[L-f], 2B = -i (Z[f] - conj Z[L-f]).
    // After v, sa holds W[f] = Oa + i Ob and sb W[L-f] = conj(Oa) + i conj(Ob).
    auto mirror = [&](int u) -> float2 {
      if (u == H2) return v[H2];
      const float2 pulled = lane_pull2(v[R - 1 - u], partner_byte);
      return special ? v[(R - u) % R] : pulled;
    };
    if (x == 0) {
#pragma unroll
      for (int u = 0; u <= H2; ++u) {
        const float2 z = v[u], zm = mirror(u);
        sa[u] = make_float2(z.x + zm.x, z.y - zm.y);
        sb[u] = make_float2(z.y + zm.y, zm.x - z.x);
      }
    } else if (x == 1) {
#pragma unroll
      for (int u = 0; u <= H2; ++u) {
        const float2 z = v[u], zm = mirror(u);
        sa[u] = cmulc(sa[u], make_float2(z.x + zm.x, z.y - zm.y));
        sb[u] = cmulc(sb[u], make_float2(z.y + zm.y, zm.x - z.x));
      }
    } else {
#pragma unroll
      for (int u = 0; u <= H2; ++u) {
        const float2 z = v[u], zm = mirror(u);
        float2 oa, ob;
        const float2 pa = cmul(sa[u], make_float2(z.x + zm.x, z.y - zm.y));
        const float2 pb = cmul(sb[u], make_float2(z.y + zm.y, zm.x - z.x));
        if constexpr (GL) {
          const float ga = gl[(s2 * (H2 + 1) + u) * R + k1];
          oa = cscale(pa, ga);
          ob = cscale(pb, ga);
        } else if constexpr (IN == IN_C32 && CG) {  // multi-level, complex gate table
          const float2 ga = reinterpret_cast<const float2*>(p.gtab)[(gta - p.gtab) + R * u];
          const float2 gb = ha == hb ? ga : reinterpret_cast<const float2*>(p.gtab)[(gtb - p.gtab) + R * u];
          oa = cmul(pa, ga);
          ob = cmul(pb, gb);
        } else if constexpr (IN == IN_C32) {  // multi-level: the gate table
          const float ga = gta[R * u];
          const float gb = ha == hb ? ga : gtb[R * u];
          oa = cscale(pa, ga);
          ob = cscale(pb, gb);
        } else {  // raw inputs, one column (single level): bin k1 + R u, from the gate itself
          const int f = k1 + R * u;
          const int fc = min(f, p.L - f);
          const bool kept = fc < p.keep;
          const float2 ga = kept ? gate_value(p.gate, p.gate_kind, p.nbins, ha, fc, f, p.L, p.scale)
                                 : make_float2(0.f, 0.f);
          const float2 gb = kept ? gate_value(p.gate, p.gate_kind, p.nbins, hb, fc, f, p.L, p.scale)
                                 : make_float2(0.f, 0.f);
          oa = cmul(pa, ga);
          ob = cmul(pb, gb);
        }
        sa[u] = make_float2(oa.x - ob.y, oa.y + ob.x);
        sb[u] = make_float2(oa.x + ob.y, ob.x - oa.y);
      }
    }
  }
  // ---- W back into this lane's own bins k2 = 0 .. R-1
#pragma unroll
  for (int u = 0; u < H2; ++u) v[u] = sa[u];
#pragma unroll
  for (int q = 0; q < H2; ++q) {
    const float2 pulled = lane_pull2(sb[H2 - 1 - q], partner_byte);
    v[H2 + q] = special ? (q == 0 ? sa[H2] : sb[H2 - q]) : pulled;
  }

  // ---- inverse, stage 2 lanes: along k2, twiddle w_N^{-k1 n}
  int k1o = k1;
  asm volatile("" : "+v"(k1o));
  dft<R, +1>(v);
#pragma unroll
  for (int n = 1; n < R; ++n) v[n] = cmul(v[n], cconj(twl[k1o * n]));
  __syncthreads();
#pragma unroll
  for (int n = 0; n < R; ++n) lds[k1 * ROW + n * ncols + col2] = v[n];
  __syncthreads();
  // ---- inverse, stage 1 lanes: along k1 -> z[t + R i], twiddle, store
#pragma unroll
  for (int k = 0; k < R; ++k) v[k] = lds[k * ROW + t1 * ncols + col1];
  // output twiddle w^-(m3 tw_mul), w = w_L, for m3 = t1 + R i, i = 4 a + j:
  // the seeds w^(t1 + R j), j < 4, times (w^(4 R))^a
  const int tw_mul = p.L1 * k2c1 + (p.L2 == 1 ? kc1 : 0);
  float2 tws[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tws[j] = p.twL[(t1 + R * j) * tw_mul];
  const float2 tw4r = p.twL[4 * R * tw_mul];
  dft<R, +1>(v);
  if (!active1) return;
  char* dst = reinterpret_cast<char*>(p.out) + batch_pair * 8;
  const uint32_t off = lane_pair * 8;
  float2 step = make_float2(1.f, 0.f);
#pragma unroll
  for (int a = 0; a < R / 4; ++a) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * a + j;
      *reinterpret_cast<float2*>(dst + i * row_pair * 8 + off) = cmul(v[i], cconj(cmul(tws[j], step)));
    }
    step = cmul(step, tw4r);
  }
}

// ------------------------- B, N = 1024, tiled input: LDS copies, persistent
//
// The square pass for R = 32 when its input is in the tiled layout and a
// workgroup holds two slots (a column and its mirror) of 4 channel pairs
// whose gate values share one head.  The arithmetic and the lane mappings
// are those of k_mid_sq; the data movement differs:
//  - each slot's input block (N rows x 4 pairs, 32 KB contiguous) is copied
//    global -> LDS by 16-byte-per-lane asynchronous loads (global_load_lds)
//    into the transpose buffer, slot 1 at a 128-byte offset so the two
//    slots' reads fall in different banks, and stage 1 reads its strided
//    elements from there;
//  - tensor x + 1's copy is issued as soon as tensor x's stage-2 reads are
//    done, and runs under its stage-2 DFT and spectral product;
//  - a workgroup takes several work items: w, w + gridDim.x, ... (with the
//    grid a multiple of 8 an item's XCD is its index mod 8, as for one item
//    per workgroup), and the next item's q copy runs under this item's last
//    inverse DFT and its stores;
//  - the copies are issued at raised wave priority (s_setprio), so that the
//    other workgroup's wave on the SIMD, busy with its transforms, does not
//    hold them back.
// The asynchronous copies write LDS, and the compiler knows that much: before
// the first LDS read after a copy it waits for every outstanding vector
// memory operation (vmcnt(0)), which at the top of an item also retires the
// previous item's U stores.  The explicit waits before the barriers that
// publish a copy are full waits as well; nothing counts operations by hand.

// CG: complex gate, read from the table in the product (no LDS copy).
// UK: the product runs over k2 = u < UK only (UK = 17: all); the host takes
// UK from the truncation, so that every bin at u >= UK is truncated.
template <bool CG, int UK = 17>
__global__ __launch_bounds__(256, 2) void k_mid_dma(MidParams p) {
  constexpr int R = 32, N = R * R, H2 = R / 2, NT = 256, ROW = R * 8 + 1;
  constexpr int kSlot = 4 * N + 16;          // float2 between the slots' blocks
  constexpr int NGL = 2 * (H2 + 1) * R;      // gate values per item
  constexpr int NGR = (NGL + NT - 1) / NT;
  extern __shared__ float2 lds[];
  float2* twl = lds + R * ROW;                         // w_N^e, e < N
  float* gl = reinterpret_cast<float*>(twl + N);       // gate values [slot][u <= R/2][k1]
  const int tid = threadIdx.x;
  // stage-1 / stage-3 identity: thread (t1, col1), col1 = slot * 4 + pair
  const int col1 = tid & 7, t1 = tid >> 3, s1 = col1 >> 2, j1 = col1 & 3;
  // stage-2 identity: thread (j2, s2, k1)
  const int j2 = tid >> 6, s2 = (tid >> 5) & 1, k1 = tid & 31, col2 = s2 * 4 + j2;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lane16 = (uint32_t)(tid & 63) * 16;
  const int ntile = p.gx * p.gy * p.gz;

  // work item -> (column pair, channel-pair block, batch), wave-uniform, and
  // its columns (scalar loads)
  auto item = [&](int t) __attribute__((always_inline)) {
    const int3 g = sharer_block_of(t, p.gx, p.gy, p.gz);
    return make_int3(__builtin_amdgcn_readfirstlane(g.x), __builtin_amdgcn_readfirstlane(g.y),
                     __builtin_amdgcn_readfirstlane(g.z));
  };
  auto copy_block = [&](const void* src, int3 blk, int2 cols) __attribute__((always_inline)) {
    const int64_t bp = (int64_t)blk.z * p.L * p.CP2;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int c = sl == 0 ? cols.x : cols.y;
      if (c < 0) continue;
      const char* g = reinterpret_cast<const char*>(src) +
                      (bp + (int64_t)((c % p.L1) * p.M + (c / p.L1) * N) * p.CP2 + (int64_t)blk.y * (N * 4)) * 8 +
                      wv * 1024;
      char* l = reinterpret_cast<char*>(lds + sl * kSlot) + wv * 1024;
#pragma unroll
      for (int q = 0; q < (N * 32) / 4096; ++q)
        __builtin_amdgcn_global_load_lds(g + q * 4096 + lane16, l + q * 4096, 16, 0, 2 /* nontemporal */);
    }
  };
  // With a truncation bound (UK < 17) the tensor loop is unrolled: each
  // tensor's product is then straight-line code and the loop's register
  // copies go, but the registers only suffice when the next item's gate
  // values are loaded during the last tensor, through 32-bit offsets from
  // the head's table.  Without a bound the unrolled loop needs more than
  // 256 VGPRs, so it stays rolled.
  constexpr bool kUnrolled = UK < 17;
  constexpr int kTensorUnroll = kUnrolled ? 3 : 1;
  auto gate_load = [&](int3 blk, int2 cols, float* gv) __attribute__((always_inline)) {
    const int hw = (2 * blk.y * 4) / p.D;  // the item's head
    const float* gb = p.gtab + (int64_t)hw * p.ncol * N;
#pragma unroll
    for (int r = 0; r < NGR; ++r) {
      const int e = min(tid + NT * r, NGL - 1);
      const int sl = e / ((H2 + 1) * R), u = (e / R) % (H2 + 1), kk = e % R;
      const int c = sl == 0 ? cols.x : cols.y;
      if constexpr (kUnrolled)
        gv[r] = gb[(uint32_t)((c >= 0 ? c : 0) * N + kk + R * u)];
      else
        gv[r] = p.gtab[((int64_t)hw * p.ncol + (c >= 0 ? c : 0)) * N + kk + R * u];
    }
  };

  int tile = blockIdx.x;
  if (tile >= ntile) return;
  int3 blk = item(tile);
  int2 cols = p.wgcols[blk.x];
  float gv[NGR];
  {
    float2 tv[N / NT];
#pragma unroll
    for (int r = 0; r < N / NT; ++r) tv[r] = p.twN[tid + NT * r];
    if constexpr (!CG) gate_load(blk, cols, gv);
    copy_block(p.in[0], blk, cols);
#pragma unroll
    for (int r = 0; r < N / NT; ++r) twl[tid + NT * r] = tv[r];
    if constexpr (!CG) {
#pragma unroll
      for (int r = 0; r < NGR; ++r)
        if (tid + NT * r < NGL) gl[tid + NT * r] = gv[r];
    }
  }
  float2 v[R];
  float2 sa[H2 + 1], sb[H2 + 1];

#pragma unroll 1
  while (true) {
    // the next item; its columns and gate values are loaded during this one
    const int next = tile + (int)gridDim.x;
    const bool more = next < ntile;
    const int3 nblk = more ? item(next) : blk;
    int2 ncols_v = make_int2(0, 0);
    // ---- this item's identity
    const bool regular = blk.x != p.selfwg;
    int ps, pk1;
    bool a_zero = false;
    if (regular) {
      ps = 1 - s2;
      pk1 = R - 1 - k1;
    } else {
      ps = s2;
      a_zero = s2 == 0;
      pk1 = a_zero ? (R - k1) % R : R - 1 - k1;
    }
    const int partner_byte = (((j2 * 64 + ps * R + pk1) & 63) << 2);
    const bool special = a_zero && k1 == 0;
    const int colid1 = s1 == 0 ? cols.x : cols.y;  // every workgroup holds two columns

#pragma unroll kTensorUnroll
    for (int x = 0; x < 3; ++x) {
      int t1o = t1;  // opaque: the 31 twiddle addresses are recomputed per tensor
      asm volatile("" : "+v"(t1o));
      // ---- stage 1 input: this wave's copies have landed, then every other
      // wave's
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      {
        const float2* raw = lds + s1 * kSlot + t1 * 4 + j1;
#pragma unroll
        for (int i = 0; i < R; ++i) v[i] = raw[i * R * 4];
      }
      // the next item's columns (a vector load: the top of the next tensor
      // waits for it), then its gate values, both used at the end of the item
      if (x == 0) ncols_v = p.wgcols[nblk.x];
      if constexpr (!CG) {
        if (x == (kUnrolled ? 2 : 1)) gate_load(nblk, ncols_v, gv);
      }
      __syncthreads();  // the blocks are read before the transpose overwrites them
      // ---- stage 1: DFT over i of x[t + R i], twiddle w_N^{t k}
      dft<R, -1>(v);
#pragma unroll
      for (int k = 1; k < R; ++k) v[k] = cmul(v[k], twl[t1o * k]);
#pragma unroll
      for (int k = 0; k < R; ++k) lds[k * ROW + t1 * 8 + col1] = v[k];
      __syncthreads();
      // ---- stage 2: DFT over t -> X[k1 + R k2]
#pragma unroll
      for (int t = 0; t < R; ++t) v[t] = lds[k1 * ROW + t * 8 + col2];
      if (x < 2) {
        __syncthreads();  // the transpose buffer is free: fetch the next tensor
        // issued at raised priority: the SIMD's other wave (the other
        // workgroup) is then in its arithmetic and would otherwise delay
        // these issues, and with them the copy the next tensor waits for
        __builtin_amdgcn_s_setprio(3);
        copy_block(p.in[x + 1], blk, cols);
        __builtin_amdgcn_s_setprio(0);
      }
      dft<R, -1>(v);
      if (p.dc != nullptr && special)  // bin 0 of column (0, 0)
        p.dc[x * p.dc_stride + (int64_t)blk.z * p.CP2 + blk.y * 4 + j2] = cscale(v[0], p.dc_scale);

      // ---- split the packed spectra and accumulate / finish the product
      // (the same arithmetic as k_mid_sq).  Regular workgroups pair every
      // bin with the partner lane and use no bin k2 = R/2 of their own; the
      // workgroup of the self-paired columns has lane k1 = 0 of column (0, 0)
      // holding its own mirrors and the self-mirrored bin k2 = R/2.
      auto product = [&](auto self_tag) __attribute__((always_inline)) {
        constexpr bool SELF = decltype(self_tag)::value;
        constexpr int NU = SELF ? H2 + 1 : H2;  // bins owned: k2 = u < NU
        auto mirror = [&](int u) -> float2 {
          if (u == H2) return v[H2];
          const float2 pulled = lane_pull2(v[R - 1 - u], partner_byte);
          if constexpr (SELF) return special ? v[(R - u) % R] : pulled;
          else return pulled;
        };
        if (x == 0) {
#pragma unroll
          for (int u = 0; u < UK && u < NU; ++u) {
            const float2 z = v[u], zm = mirror(u);
            sa[u] = make_float2(z.x + zm.x, z.y - zm.y);
            sb[u] = make_float2(z.y + zm.y, zm.x - z.x);
          }
        } else if (x == 1) {
#pragma unroll
          for (int u = 0; u < UK && u < NU; ++u) {
            const float2 z = v[u], zm = mirror(u);
            sa[u] = cmulc(sa[u], make_float2(z.x + zm.x, z.y - zm.y));
            sb[u] = cmulc(sb[u], make_float2(z.y + zm.y, zm.x - z.x));
          }
        } else {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            if (u >= UK) {  // every bin from here on truncated
              sa[u] = sb[u] = make_float2(0.f, 0.f);
              continue;
            }
            const float2 z = v[u], zm = mirror(u);
            const float2 pa = cmul(sa[u], make_float2(z.x + zm.x, z.y - zm.y));
            const float2 pb = cmul(sb[u], make_float2(z.y + zm.y, zm.x - z.x));
            float2 oa, ob;
            if constexpr (CG) {
              const int c2 = s2 == 0 ? cols.x : cols.y;
              const float2 g = reinterpret_cast<const float2*>(p.gtab)
                  [((int64_t)((2 * blk.y * 4) / p.D) * p.ncol + (c2 >= 0 ? c2 : 0)) * N + k1 + R * u];
              oa = cmul(pa, g);
              ob = cmul(pb, g);
            } else {
              const float g = gl[(s2 * (H2 + 1) + u) * R + k1];
              oa = cscale(pa, g);
              ob = cscale(pb, g);
            }
            sa[u] = make_float2(oa.x - ob.y, oa.y + ob.x);
            sb[u] = make_float2(oa.x + ob.y, ob.x - oa.y);
          }
        }
      };
      if (regular)
        product(std::false_type{});
      else
        product(std::true_type{});
    }
    // ---- W back into this lane's own bins k2 = 0 .. R-1
#pragma unroll
    for (int u = 0; u < H2; ++u) v[u] = sa[u];
    if (regular) {
#pragma unroll
      for (int q = 0; q < H2; ++q) v[H2 + q] = lane_pull2(sb[H2 - 1 - q], partner_byte);
    } else {
#pragma unroll
      for (int q = 0; q < H2; ++q) {
        const float2 pulled = lane_pull2(sb[H2 - 1 - q], partner_byte);
        v[H2 + q] = special ? (q == 0 ? sa[H2] : sb[H2 - q]) : pulled;
      }
    }
    // ---- inverse, stage 2 lanes: along k2, twiddle w_N^{-k1 n}
    int k1o = k1;
    asm volatile("" : "+v"(k1o));
    dft<R, +1>(v);
#pragma unroll
    for (int n = 1; n < R; ++n) v[n] = cmul(v[n], cconj(twl[k1o * n]));
    __syncthreads();
#pragma unroll
    for (int n = 0; n < R; ++n) lds[k1 * ROW + n * 8 + col2] = v[n];
    // the next item's gate values (every wave has read this item's)
    if constexpr (!CG) {
#pragma unroll
      for (int r = 0; r < NGR; ++r)
        if (tid + NT * r < NGL) gl[tid + NT * r] = gv[r];
    }
    // output twiddle w^-(m3 tw_mul), w = w_L, for m3 = t1 + R i, i = 4 a + j:
    // the seeds w^(t1 + R j), j < 4, times (w^(4 R))^a; loaded before the
    // next item's copy so that waiting for them does not wait for it
    const int kc1 = colid1 % p.L1, k2c1 = colid1 / p.L1;
    const int tw_mul = p.L1 * k2c1 + (p.L2 == 1 ? kc1 : 0);
    float2 tws[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tws[j] = p.twL[(t1 + R * j) * tw_mul];
    float2 tw4r = p.twL[4 * R * tw_mul];
    __syncthreads();
    // ---- inverse, stage 1 lanes: along k1 -> z[t + R i]
#pragma unroll
    for (int k = 0; k < R; ++k) v[k] = lds[k * ROW + t1 * 8 + col1];
    // the seeds have arrived before the copy is issued, so that nothing
    // after it waits on the copy
    asm volatile("" : "+v"(tws[0]), "+v"(tws[1]), "+v"(tws[2]), "+v"(tws[3]), "+v"(tw4r));
    asm volatile("" : "+v"(ncols_v));
    const int2 ncols = make_int2(__builtin_amdgcn_readfirstlane(ncols_v.x), __builtin_amdgcn_readfirstlane(ncols_v.y));
    __syncthreads();  // the transpose buffer is free: fetch the next item's q
    __builtin_amdgcn_s_setprio(3);
    if (more) copy_block(p.in[0], nblk, ncols);
    __builtin_amdgcn_s_setprio(0);
    dft<R, +1>(v);
    // U in row layout: element i of this lane is token row m3 = t1 + R i
    const int cp1 = blk.y * 4 + j1;
    const uint32_t lane_pair = (uint32_t)((kc1 * p.M + k2c1 * N + t1) * p.CP2 + cp1);
    const int64_t row_pair = (int64_t)R * p.CP2;
    char* dst = reinterpret_cast<char*>(p.out) + (int64_t)blk.z * p.L * p.CP2 * 8;
    const uint32_t off = lane_pair * 8;
    float2 step = make_float2(1.f, 0.f);
#pragma unroll
    for (int a = 0; a < R / 4; ++a) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * a + j;
        *reinterpret_cast<float2*>(dst + i * row_pair * 8 + off) = cmul(v[i], cconj(cmul(tws[j], step)));
      }
      step = cmul(step, tw4r);
    }
    if (!more) break;
    tile = next;
    blk = nblk;
    cols = ncols;
  }
}

// ------------------------------ single-pass column kernel, L = RA * RB * RC
//
// For L up to 8192 a channel pair's whole column fits in LDS, so one
// workgroup runs the whole spectral path for CPT neighbouring channel pairs
// of one batch element: q, k and v read once (CPT * 8 bytes of every row),
// three forward transforms, the spectral product, the inverse, y written
// once.  The norm runs as its own pass, since it needs every channel of a
// token.  The L-point transform is three register-DFT stages joined by two
// LDS exchanges (a four-step split applied twice):
//   n = a + TA jA (TA = RB RC),  a = b + RC jB,  f = kA + RA (kB + RB kC)
//   A  thread a < TA:             DFT_RA over jA, times w_L^{a kA}
//   B  thread b + RC kA < TB:     DFT_RB over jB, times w_L^{RA b kB}
//   C  thread kA + RA kB < TC:    DFT_RC over b  -> X[f], f = t + TC kC
// (TB = L / RB, TC = L / RC).  Per pair, in binary32 pairs, the A -> B
// exchange sits at kA TA + a and the B -> C exchange at (kA + RA kB)(RC + 1)
// + b: the pad of one element per C thread makes both the strided writes
// and the transposed reads hit distinct banks.  Bins go through LDS in
// natural order for the mirror reads of the product and for the inverse.
// A wave's lanes take 16 consecutive column threads of each of its pairs,
// and the pair regions are REGION = 16 (mod 32) elements apart, so every
// exchange touches distinct banks per 16 lanes (32 banks) and per 32 lanes
// (64 banks).  Twiddle powers come from one table value per stage by repeated
// multiplication (at most RA - 2 products, a few units of binary32
// rounding).
//
// Measured on MI355X at L = 4096 (B = 4, H*D = 512): about 4100 VALU
// instructions per thread (28 us of issue per CU), 10 us of LDS exchanges and
// the HBM traffic do not overlap, since one 1024-thread workgroup per CU
// moves through them in lockstep; loading the next tensor during a transform
// (registers) gained nothing there and is not done.

template <int RA_, int RB_, int RC_, int CPT>
struct ColCfg {
  static constexpr int RA = RA_, RB = RB_, RC = RC_;
  static constexpr int N = RA * RB * RC;
  static constexpr int TA = N / RA, TB = N / RB, TC = N / RC;
  static constexpr int TP = TA > TB ? (TA > TC ? TA : TC) : (TB > TC ? TB : TC);
  static constexpr int THREADS = CPT * TP;
  static constexpr int VMAX = RA > RB ? (RA > RC ? RA : RC) : (RB > RC ? RB : RC);
  static constexpr int NH = RC / 2 + 1;  // product slots of a C thread
  static constexpr int region() {
    int r = N + TC;
    while (r % 32 != 16) ++r;
    return r;
  }
  static constexpr int REGION = region();
  static constexpr size_t LDS_BYTES = (size_t)CPT * REGION * sizeof(float2);
  // waves per SIMD to allow: two workgroups per CU when their LDS fits
  static constexpr int WAVES_PER_EU = (THREADS / 256) * (2 * LDS_BYTES <= 160 * 1024 ? 2 : 1);
  static_assert(RC % 2 == 0, "the product pairs bins t + TC i with i < RC / 2");
  static_assert(THREADS <= 1024 && THREADS % (16 * CPT) == 0, "one workgroup of whole lane groups");
};

struct ColParams {
  const void* in[3];   // q, k, v: [B][L][CP2] channel pairs (storage kind IN)
  const void* x;       // residual (storage kind IN) added to y before the store, or null
  float2* out;         // y, or x + y: [B][L][CP2] binary32 pairs
  const float* gate;   // [H][nbins] (pairs for a complex gate)
  const float2* tw;    // tw[e] = exp(-2 pi i e / L), e < L
  int gate_kind;
  int CP2, D, keep, nbins;
  float scale;         // 1 / (8 L^2): the mix's 1/L, the inverse's 1/L, (1/2)^3 of the split
  // chunked mix: bin 0 of each tensor times dc_scale to dc[x * dc_stride + b * CP2 + pair]
  float2* dc;
  int64_t dc_stride;
  float dc_scale;
};

// v[k] *= w^k, k = 1 .. R - 1.  The base is passed through an empty asm
// statement so that the powers are recomputed at each use: otherwise the
// compiler merges the identical powers of every transform of the kernel and
// keeps all of them live across it, which costs more registers than the
// multiplications.
template <int R>
__device__ __forceinline__ void twiddle_powers(float2* v, float2 w) {
  asm volatile("" : "+v"(w.x), "+v"(w.y));
  float2 t = w;
#pragma unroll
  for (int k = 1; k < R; ++k) {
    v[k] = cmul(v[k], t);
    if (k + 1 < R) t = cmul(t, w);
  }
}

// The L-point transform of one pair's column.  On entry thread t < TA holds
// v[j] = x[t + TA j]; on exit thread t < TC holds v[kC] = X[t + TC kC].  The
// caller makes sure the region is free on entry; on exit the C stage's LDS
// reads are issued (the caller synchronises before the region is reused).
template <class C, int SIGN>
__device__ __forceinline__ void col_fft(float2 (&v)[C::VMAX], float2* col, int t, float2 wa,
                                        float2 wb) {
  if (t < C::TA) {
    dft<C::RA, SIGN>(v);
    twiddle_powers<C::RA>(v, wa);
#pragma unroll
    for (int k = 0; k < C::RA; ++k) col[k * C::TA + t] = v[k];
  }
  __syncthreads();
  const int b = t % C::RC, kA = t / C::RC;
  if (t < C::TB) {
#pragma unroll
    for (int j = 0; j < C::RB; ++j) v[j] = col[kA * C::TA + b + C::RC * j];
  }
  __syncthreads();
  if (t < C::TB) {
    dft<C::RB, SIGN>(v);
    twiddle_powers<C::RB>(v, wb);
#pragma unroll
    for (int k = 0; k < C::RB; ++k) col[(kA + C::RA * k) * (C::RC + 1) + b] = v[k];
  }
  __syncthreads();
  if (t < C::TC) {
#pragma unroll
    for (int j = 0; j < C::RC; ++j) v[j] = col[t * (C::RC + 1) + j];
    dft<C::RC, SIGN>(v);
  }
}

template <int RA, int RB, int RC, int CPT, int IN>
__global__ __launch_bounds__((ColCfg<RA, RB, RC, CPT>::THREADS), (ColCfg<RA, RB, RC, CPT>::WAVES_PER_EU))
void k_col(ColParams p) {
  using C = ColCfg<RA, RB, RC, CPT>;
  constexpr int N = C::N;
  extern __shared__ float2 lds[];
  // one-dimensional grid: item = pair block + nblk * batch element, XCD-grouped
  const int nblk = (p.CP2 + CPT - 1) / CPT;
  const int item = xcd_grouped_block().x;
  // lanes: 16 consecutive column threads per pair, the CPT pairs side by side
  const int tid = threadIdx.x;
  const int pr = (tid >> 4) % CPT, t = (tid & 15) + 16 * (tid / (16 * CPT));
  const int cp = (item % nblk) * CPT + pr;
  const bool live = cp < p.CP2;  // a ragged last block computes on zeros and stores nothing
  const int64_t b = item / nblk;
  float2* col = lds + pr * C::REGION;
  // rows of this batch element: a uniform base per row group and one 32-bit
  // lane offset (a batch element spans L * CP2 pairs, below 2^29)
  const int64_t gbase = b * N * p.CP2;
  const uint32_t rowb = (uint32_t)p.CP2 * pair_bytes<IN>();  // bytes per row, input
  // Every row load is issued by every lane, from a clamped in-bounds address
  // (row t or 0, pair cp or CP2 - 1), and zeroed afterwards where it is not
  // wanted: loads under a branch would leave the number of younger loads in
  // flight unknown, and the wait for the oldest would then drain them all.
  const int cpc = live ? cp : p.CP2 - 1;
  const uint32_t loff_a = ((uint32_t)(t < C::TA ? t : 0) * p.CP2 + cpc) * pair_bytes<IN>();
  const uint32_t loff_c = ((uint32_t)(t < C::TC ? t : 0) * p.CP2 + cpc) * pair_bytes<IN>();
  const bool want_a = t < C::TA && live;

  // twiddle bases, loaded before the rows: a wait for them then drains nothing else
  const float2 wa = p.tw[t < C::TA ? t : 0];
  const float2 wb = p.tw[C::RA * (t % C::RC)];

  float2 nxt[C::RA];
  auto load_rows = [&](const void* src) __attribute__((always_inline)) {
    const char* ub = static_cast<const char*>(src) + gbase * pair_bytes<IN>();
    __builtin_amdgcn_s_setprio(3);  // ahead of other waves' transforms (about 1 us at 4096)
#pragma unroll
    for (int j = 0; j < C::RA; ++j) {
      const float2 r = load_pair_c<IN>(ub + (size_t)j * C::TA * rowb, loff_a);
      nxt[j] = want_a ? r : make_float2(0.f, 0.f);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  load_rows(p.in[0]);

  // mirror bin L - f of f = t + TC i (i < RC/2) at mcol[TC (RC/2 - 1 - i)],
  // a base and positive immediate offsets; f = 0 and f = L/2 are their own
  // mirrors
  float2* const mcol = col + (N - t - C::TC * (RC / 2 - 1));
  auto mirror_at = [](float2* mc, float2* c, int t, int i) __attribute__((always_inline)) -> float2* {
    if (i == RC / 2) return c + N / 2;
    if (i == 0 && t == 0) return c;
    return mc + C::TC * (RC / 2 - 1 - i);
  };
  float2 v[C::VMAX];
  float2 sa[C::NH], sb[C::NH];
  const int ha = live ? (2 * cp) / p.D : 0, hb = live ? (2 * cp + 1) / p.D : 0;  // heads
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    if (x > 0) load_rows(p.in[x]);
#pragma unroll
    for (int j = 0; j < C::RA; ++j) v[j] = nxt[j];
    if (x > 0) __syncthreads();  // the previous tensor's mirror reads are done
    col_fft<C, -1>(v, col, t, wa, wb);
    __syncthreads();  // every C-stage read is done before the bins overwrite the region
    if (t < C::TC) {
#pragma unroll
      for (int i = 0; i < RC; ++i) col[t + C::TC * i] = v[i];
    }
    if (p.dc != nullptr && t == 0 && live)  // bin 0
      p.dc[x * p.dc_stride + b * p.CP2 + cp] = cscale(v[0], p.dc_scale);
    __syncthreads();
    if (t < C::TC) {
      // bin pairs (f, L - f), f = t + TC i for i < RC/2, and f = L/2 (t = 0):
      // 2A = Z[f] + conj Z[L-f], 2B = -i (Z[f] - conj Z[L-f])
#pragma unroll
      for (int i = 0; i < C::NH; ++i) {
        if (i == RC / 2 && t != 0) continue;
        const int f = t + C::TC * i;
        const float2 z = v[i], zm = *mirror_at(mcol, col, t, i);
        const float2 A = make_float2(z.x + zm.x, z.y - zm.y);
        const float2 Bv = make_float2(z.y + zm.y, zm.x - z.x);
        if (x == 0) {
          sa[i] = A;
          sb[i] = Bv;
        } else if (x == 1) {
          sa[i] = cmulc(sa[i], A);
          sb[i] = cmulc(sb[i], Bv);
        } else {
          float2 ga = make_float2(0.f, 0.f), gb = ga;
          if (f < p.keep) {
            ga = gate_value(p.gate, p.gate_kind, p.nbins, ha, f, f, N, p.scale);
            gb = gate_value(p.gate, p.gate_kind, p.nbins, hb, f, f, N, p.scale);
          }
          sa[i] = cmul(cmul(sa[i], A), ga);
          sb[i] = cmul(cmul(sb[i], Bv), gb);
        }
      }
    }
  }
  __syncthreads();  // every mirror read is done
  if (t < C::TC) {
    // W[f] = Oa + i Ob, W[L-f] = conj(Oa) + i conj(Ob)
#pragma unroll
    for (int i = 0; i < C::NH; ++i) {
      if (i == RC / 2 && t != 0) continue;
      const float2 oa = sa[i], ob = sb[i];
      col[t + C::TC * i] = make_float2(oa.x - ob.y, oa.y + ob.x);
      *mirror_at(mcol, col, t, i) = make_float2(oa.x + ob.y, ob.x - oa.y);
    }
  }
  __syncthreads();
  if (t < C::TA) {
#pragma unroll
    for (int j = 0; j < RA; ++j) v[j] = col[t + C::TA * j];
  }
  __syncthreads();  // read before the A stage overwrites the region
  // the residual rows this thread stores, loaded while the inverse runs
  float2 xr[RC];
  const bool addx = p.x != nullptr;
  if (addx) {
    const char* xb = static_cast<const char*>(p.x) + gbase * pair_bytes<IN>();
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int i = 0; i < RC; ++i) xr[i] = load_pair_c<IN>(xb + (size_t)i * C::TC * rowb, loff_c);
    __builtin_amdgcn_s_setprio(0);
  }
  col_fft<C, +1>(v, col, t, cconj(wa), cconj(wb));
  if (t < C::TC && live) {
    char* ob = reinterpret_cast<char*>(p.out + gbase);
    const uint32_t orow = (uint32_t)p.CP2 * sizeof(float2);
    const uint32_t ooff = ((uint32_t)t * p.CP2 + cp) * sizeof(float2);
#pragma unroll
    for (int i = 0; i < RC; ++i)
      *reinterpret_cast<float2*>(ob + (size_t)i * C::TC * orow + ooff) = addx ? cadd(v[i], xr[i]) : v[i];
  }
}

// ------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// C1 token statistics.  Each lane holds NV per-token values (NV a power of
// two <= 64); recursive halving over lane bits 32, 16, ... leaves lane l with
// the wave's total for token l >> (6 - log2 NV), and the remaining lane bits
// are summed by plain butterflies.  Then the waves' totals meet in LDS.
template <int NV, int O>
__device__ __forceinline__ void halve_sums(float* vals, int lane) {
  if constexpr (O == 0) {
    return;
  } else if constexpr (NV > 1) {
    constexpr int half = NV / 2;
    const bool up = (lane & O) != 0;
#pragma unroll
    for (int q = 0; q < half; ++q) {
      const float mine = up ? vals[half + q] : vals[q];
      const float other = up ? vals[q] : vals[half + q];
      vals[q] = mine + __shfl_xor(other, O, 64);
    }
    halve_sums<half, O / 2>(vals, lane);
  } else {
    vals[0] += __shfl_xor(vals[0], O, 64);
    halve_sums<1, O / 2>(vals, lane);
  }
}

template <int Rp>
__device__ __forceinline__ float wave_token_sums(float (&t)[Rp], int lane) {
  halve_sums<Rp, 32>(t, lane);
  return t[0];
}

constexpr int next_pow2(int r) { return r <= 1 ? 1 : 2 * next_pow2((r + 1) / 2); }
constexpr int ilog2(int r) { return r <= 1 ? 0 : 1 + ilog2(r / 2); }

// The local branch joins y: y + y_loc, or with per-channel weights
// g = mix[2 cp], mix[2 cp + 1] the gated form g y + (1 - g) y_loc.
__device__ __forceinline__ float2 join_branches(float2 y, float2 yl, bool gated, float2 g) {
  if (!gated) return cadd(y, yl);
  return make_float2(g.x * y.x + (1.0f - g.x) * yl.x, g.y * y.y + (1.0f - g.y) * yl.y);
}

// ----------------------------------------- C1: inverse L1 DFT (+ LayerNorm)
//
// One thread per (b, m, pair): R = L1 loads U[b][k1][m][pair], an inverse
// R-point DFT gives tokens t = n1 M + m.  With FUSE the workgroup is exactly
// the CP2 pairs of one (b, m), so every token's H*D channels are in the
// workgroup: residual add, two-pass mean / variance over the channels, affine,
// store (PRE: the statistics of y alone, and x added after the affine step).
// Without FUSE it stores y (binary32) for a separate LayerNorm pass.

struct FinalParams {
  const float2* U;
  const void* x;
  const float* gamma;
  const float* beta;
  void* out;  // dtype out, or float y when not fused
  int64_t M, CP2, L;
  int64_t lines;  // B * M * CP2
  float inv_c;
  float eps;
  const float2* yblk;  // chunked mix: [B][CP2] term added to every token of batch (block) b, or null
  const float2* yloc;  // local branch: [B][L][CP2] term added to y, or null
  const float* mix;    // with yloc: per-channel weight g, y <- g y + (1 - g) y_loc; null: y + y_loc
  int rms;             // 1: RMSNorm (no mean subtracted), 0: LayerNorm
};

template <int R, int DT, bool FUSE, bool PRE = false>
__global__ __launch_bounds__(256) void k_final(FinalParams p) {
  constexpr int Rp = next_pow2(R);
  // fused: one workgroup per (b, m) with exactly CP2 threads; else a flat grid
  const int64_t line = FUSE ? (int64_t)blockIdx.x * p.CP2 + threadIdx.x
                            : (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (!FUSE && line >= p.lines) return;
  const int64_t cp = line % p.CP2;
  const int64_t bm = line / p.CP2;  // b * M + m
  const int64_t m = bm % p.M;
  const int64_t b = bm / p.M;

  float2 z[R];
  const int64_t ubase = (b * R * p.M + m) * p.CP2 + cp;
#pragma unroll
  for (int r = 0; r < R; ++r) z[r] = load_nt(p.U + ubase + (int64_t)r * p.M * p.CP2);
  dft<R, +1>(z);
  if (p.yblk != nullptr) {  // chunked mix: the block term, the same for the R tokens
    const float2 yb = p.yblk[b * p.CP2 + cp];
#pragma unroll
    for (int r = 0; r < R; ++r) z[r] = cadd(z[r], yb);
  }

  // token t = n1 M + m of batch b sits at pair offset ((b L) + t) CP2 + cp
  const int64_t obase = (b * p.L + m) * p.CP2 + cp;
  const int64_t ostep = p.M * p.CP2;
  if (p.yloc != nullptr) {  // local branch: its output joins y
    const bool gated = p.mix != nullptr;
    const float2 g = gated ? make_float2(p.mix[2 * cp], p.mix[2 * cp + 1]) : make_float2(1.f, 1.f);
#pragma unroll
    for (int r = 0; r < R; ++r) z[r] = join_branches(z[r], load_nt(p.yloc + obase + r * ostep), gated, g);
  }
  if constexpr (!FUSE) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float2* yp = reinterpret_cast<float2*>(p.out) + obase + r * ostep;
      *yp = z[r];
    }
  } else {
    __shared__ float red[4][Rp];
    __shared__ float tot[Rp];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    if constexpr (!PRE) {  // post-norm: the statistics are those of x + y
#pragma unroll
      for (int r = 0; r < R; ++r) z[r] = cadd(z[r], load_pair<DT>(p.x, obase + r * ostep));
    }

    float t[Rp];
    float mean[R], rstd[R];
    // pass 1: mean (times 0 for an RMSNorm, which subtracts none)
    {
#pragma unroll
      for (int r = 0; r < Rp; ++r) t[r] = r < R ? z[r].x + z[r].y : 0.f;
      float s = wave_token_sums<Rp>(t, lane);
      if ((lane & ((64 / Rp) - 1)) == 0) red[wave][lane / (64 / Rp)] = s;
      __syncthreads();
      if (threadIdx.x < Rp) {
        float a = 0.f;
        for (int w = 0; w < nw; ++w) a += red[w][threadIdx.x];
        tot[threadIdx.x] = a * (p.rms ? 0.f : p.inv_c);
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) mean[r] = tot[r];
      __syncthreads();
    }
    // pass 2: biased variance of the centred values (mean square for RMSNorm)
#pragma unroll
    for (int r = 0; r < Rp; ++r) {
      if (r < R) {
        const float dx = z[r].x - mean[r], dy = z[r].y - mean[r];
        t[r] = dx * dx + dy * dy;
      } else {
        t[r] = 0.f;
      }
    }
    {
      float s = wave_token_sums<Rp>(t, lane);
      if ((lane & ((64 / Rp) - 1)) == 0) red[wave][lane / (64 / Rp)] = s;
      __syncthreads();
      if (threadIdx.x < Rp) {
        float a = 0.f;
        for (int w = 0; w < nw; ++w) a += red[w][threadIdx.x];
        tot[threadIdx.x] = 1.0f / sqrtf(a * p.inv_c + p.eps);
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) rstd[r] = tot[r];
    }
    const float g0 = p.gamma[2 * cp], g1 = p.gamma[2 * cp + 1];
    const float b0 = p.beta[2 * cp], b1 = p.beta[2 * cp + 1];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float2 o = make_float2((z[r].x - mean[r]) * rstd[r] * g0 + b0,
                             (z[r].y - mean[r]) * rstd[r] * g1 + b1);
      if constexpr (PRE) o = cadd(o, load_pair<DT>(p.x, obase + r * ostep));  // x + LN(y)
      store_pair<DT>(p.out, obase + r * ostep, o);
    }
  }
}

// C1 with the R-point inverse DFT split over lanes l and l^32 (R = 48, 64),
// fused with the residual and the LayerNorm.  One workgroup per (b, m) with
// 2 CP2 threads: wave w, lane h * 32 + c serves pair 32 w + c; half h loads
// the rows k1 = 2a + h and transforms them (R/2 points), and join_swap
// finishes the radix-2 step, leaving half h with R/2 of the R tokens (slot j
// holds token tok(j)).  Half the registers of k_final, so four times the
// waves per CU.  Token sums: recursive halving over the 32 lanes of a half
// (lane c ends with the half-wave total of slot c), then the waves' totals
// meet in LDS.  Needs CP2 % 32 == 0 and CP2 <= 256.
// ADD: 0 nothing more, 1 the chunked mix's block term, 2 the local branch.
template <int R, int DT, bool PRE = false, int ADD = 0>
__global__ __launch_bounds__(512, 4) void k_final_split(FinalParams p) {
  constexpr int R2 = R / 2;
  constexpr int T2 = next_pow2(R2);  // 32: token slots per half
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int nw = blockDim.x >> 6;
  const int64_t cp = (int64_t)wave * 32 + c;
  const int64_t bm = blockIdx.x;  // b * M + m
  const int64_t m = bm % p.M;
  const int64_t b = bm / p.M;
  __shared__ float red[8][2 * T2];
  __shared__ float s_mean[2 * T2], s_rstd[2 * T2];

  float2 z[R2];
  {
    const float2* u = p.U + ((b * R + h) * p.M + m) * p.CP2 + cp;
    const int64_t rs = 2 * p.M * p.CP2;  // rows 2a + h
    __builtin_amdgcn_s_setprio(3);  // the loads ahead of other waves' arithmetic
#pragma unroll
    for (int a = 0; a < R2; ++a) z[a] = load_nt(u + a * rs);
    __builtin_amdgcn_s_setprio(0);
  }
  dft<R2, +1>(z);
  join_swap<R, +1>(z, h);
  if constexpr (ADD == 1) {  // chunked mix: the block term, the same for every token here
    const float2 yb = p.yblk[b * p.CP2 + cp];
#pragma unroll
    for (int a = 0; a < R2; ++a) z[a] = cadd(z[a], yb);
  }
  // slot j of half h holds token n1 = tok(j) (join_swap's output order);
  // token t = n1 M + m of batch b sits at pair offset ((b L) + t) CP2 + cp
  constexpr int Q = R / 4;
  auto tok = [&](int j) { return (j < Q ? j : j + Q) + Q * h; };
  const int64_t ostep = p.M * p.CP2;
  const int64_t obase = (b * p.L + m) * p.CP2 + cp + (int64_t)(Q * h) * ostep;
  auto toff = [&](int j) { return (int64_t)(j < Q ? j : j + Q) * ostep; };  // tok(j) - Q h
  if constexpr (ADD == 2) {  // local branch: its output joins y
    const bool gated = p.mix != nullptr;
    const float2 gw = gated ? make_float2(p.mix[2 * cp], p.mix[2 * cp + 1]) : make_float2(1.f, 1.f);
#pragma unroll
    for (int g = 0; g < R2; g += 8) {
#pragma unroll
      for (int j = g; j < g + 8 && j < R2; ++j)
        z[j] = join_branches(z[j], load_nt(p.yloc + obase + toff(j)), gated, gw);
      asm volatile("" ::: "memory");
    }
  }
  // residual, loaded in groups of 8 so that the loads in flight fit the
  // register budget of four waves per SIMD
  if constexpr (!PRE) {  // post-norm: the statistics are those of x + y
#pragma unroll
    for (int g = 0; g < R2; g += 8) {
#pragma unroll
      for (int j = g; j < g + 8 && j < R2; ++j) z[j] = cadd(z[j], load_pair<DT>(p.x, obase + toff(j)));
      asm volatile("" ::: "memory");
    }
  }

  // per-token sums over the workgroup's pairs: lane c ends with slot c's total
  const float mean_w = p.rms ? 0.f : p.inv_c;  // an RMSNorm subtracts no mean
  auto token_sums = [&](float (&t)[T2], float* dst, bool is_var) __attribute__((always_inline)) {
    halve_sums<T2, 16>(t, lane);
    if (c < R2) red[wave][tok(c)] = t[0];
    __syncthreads();
    if (tid < R) {
      float a = 0.f;
      for (int w = 0; w < nw; ++w) a += red[w][tid];
      dst[tid] = is_var ? 1.0f / sqrtf(a * p.inv_c + p.eps) : a * mean_w;
    }
    __syncthreads();
  };
  {  // the mean, times 0 for an RMSNorm (straight-line code either way)
    float t[T2];
#pragma unroll
    for (int n = 0; n < T2; ++n) t[n] = n < R2 ? z[n].x + z[n].y : 0.f;
    token_sums(t, s_mean, false);
  }
  {
    float t[T2];
#pragma unroll
    for (int n = 0; n < T2; ++n) {
      if (n < R2) {
        const float mu = s_mean[tok(n)];
        const float dx = z[n].x - mu, dy = z[n].y - mu;
        t[n] = dx * dx + dy * dy;
      } else {
        t[n] = 0.f;
      }
    }
    token_sums(t, s_rstd, true);
  }
  const float g0 = p.gamma[2 * cp], g1 = p.gamma[2 * cp + 1];
  const float b0 = p.beta[2 * cp], b1 = p.beta[2 * cp + 1];
#pragma unroll
  for (int n = 0; n < R2; ++n) {
    const float mu = s_mean[tok(n)], rs = s_rstd[tok(n)];
    float2 o = make_float2((z[n].x - mu) * rs * g0 + b0, (z[n].y - mu) * rs * g1 + b1);
    if constexpr (PRE) o = cadd(o, load_pair<DT>(p.x, obase + toff(n)));  // x + LN(y)
    store_pair<DT>(p.out, obase + toff(n), o);
  }
}

// ------------------------------------------------ standalone LayerNorm
//
// One wave per token: lanes stride over the token's channel pairs (ITS
// pairs per lane, CP2 <= 64 ITS; H*D <= 4096), z = x + y kept in registers,
// two-pass statistics with wave butterflies, affine, store (PRE: z = y, and
// x is added after the affine step).  ITS is the smallest power of two that
// covers the token, so the registers (and the occupancy) follow H*D.

struct NormParams {
  const float2* y;
  const void* x;  // residual; null when y already holds x + y (post-norm only)
  const float* gamma;
  const float* beta;
  void* out;
  int64_t ntok, CP2;
  float inv_c, eps;
  const float2* yblk;  // chunked mix: [ntok / Lb][CP2] block term added to y, or null
  int64_t Lb;          // tokens per block
  const float2* yloc;  // local branch: [ntok][CP2] term added to y, or null
  const float* mix;    // with yloc: per-channel weight g, y <- g y + (1 - g) y_loc; null: y + y_loc
  int rms;             // 1: RMSNorm (no mean subtracted), 0: LayerNorm
};

template <int DT, bool PRE, int ITS>
__global__ __launch_bounds__(256) void k_layernorm(NormParams p) {
  constexpr int MAXIT = ITS;
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (tok >= p.ntok) return;
  const int64_t base = tok * p.CP2;
  float2 z[MAXIT];
  float s = 0.f;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int64_t c = lane + 64 * it;
    if (c < p.CP2) {
      z[it] = load_nt(p.y + base + c);
      if (p.yblk != nullptr) z[it] = cadd(z[it], p.yblk[(tok / p.Lb) * p.CP2 + c]);
      if (p.yloc != nullptr) {
        const bool gated = p.mix != nullptr;
        const float2 g = gated ? make_float2(p.mix[2 * c], p.mix[2 * c + 1]) : make_float2(1.f, 1.f);
        z[it] = join_branches(z[it], load_nt(p.yloc + base + c), gated, g);
      }
      if (!PRE && p.x != nullptr) z[it] = cadd(z[it], load_pair<DT>(p.x, base + c));
      s += z[it].x + z[it].y;
    }
  }
  const float mean = p.rms ? 0.f : wave_sum(s) * p.inv_c;  // an RMSNorm subtracts none
  float q = 0.f;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int64_t c = lane + 64 * it;
    if (c < p.CP2) {
      const float dx = z[it].x - mean, dy = z[it].y - mean;
      q += dx * dx + dy * dy;
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * p.inv_c + p.eps);
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int64_t c = lane + 64 * it;
    if (c < p.CP2) {
      float2 o = make_float2((z[it].x - mean) * rstd * p.gamma[2 * c] + p.beta[2 * c],
                             (z[it].y - mean) * rstd * p.gamma[2 * c + 1] + p.beta[2 * c + 1]);
      if constexpr (PRE) o = cadd(o, load_pair<DT>(p.x, base + c));  // x + LN(y)
      store_pair<DT>(p.out, base + c, o);
    }
  }
}

// The same with two channel pairs per lane (CP2 even): 16-byte loads of y
// and of gamma / beta, lanes over pair couples c = lane + 64 it (pairs 2c,
// 2c + 1), CP2 <= 128 ITS.
template <int DT>
__device__ __forceinline__ float4 load_pair2(const void* base, int64_t off2) {
  if constexpr (DT == IN_BF16) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base) + off2);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  } else {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base) + off2);
    return make_float4(v.x, v.y, v.z, v.w);
  }
}

template <int DT>
__device__ __forceinline__ void store_pair2(void* base, int64_t off2, float4 v) {
  if constexpr (DT == IN_BF16) {
    const uint2 u = make_uint2(f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16),
                               f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16));
    __builtin_nontemporal_store(u.x, &(reinterpret_cast<uint2*>(base) + off2)->x);
    __builtin_nontemporal_store(u.y, &(reinterpret_cast<uint2*>(base) + off2)->y);
  } else {
    float4* p = reinterpret_cast<float4*>(base) + off2;
    __builtin_nontemporal_store(v.x, &p->x);
    __builtin_nontemporal_store(v.y, &p->y);
    __builtin_nontemporal_store(v.z, &p->z);
    __builtin_nontemporal_store(v.w, &p->w);
  }
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

template <int DT, bool PRE, int ITS>
__global__ __launch_bounds__(256) void k_layernorm2(NormParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (tok >= p.ntok) return;
  const int64_t C2 = p.CP2 / 2;  // pair couples per token
  const int64_t base = tok * C2;
  const float4* y4 = reinterpret_cast<const float4*>(p.y);
  float4 z[ITS];
  float s = 0.f;
#pragma unroll
  for (int it = 0; it < ITS; ++it) {
    const int64_t c = lane + 64 * it;
    if (c < C2) {
      z[it] = load_pair2<IN_F32>(y4, base + c);
      if (p.yblk != nullptr) {
        const float4 yb = reinterpret_cast<const float4*>(p.yblk)[(tok / p.Lb) * C2 + c];
        z[it] = add4(z[it], yb);
      }
      if (p.yloc != nullptr) {
        const float4 yl = load_pair2<IN_F32>(p.yloc, base + c);
        if (p.mix != nullptr) {
          const float4 g = reinterpret_cast<const float4*>(p.mix)[c];
          z[it] = make_float4(g.x * z[it].x + (1.0f - g.x) * yl.x, g.y * z[it].y + (1.0f - g.y) * yl.y,
                              g.z * z[it].z + (1.0f - g.z) * yl.z, g.w * z[it].w + (1.0f - g.w) * yl.w);
        } else {
          z[it] = add4(z[it], yl);
        }
      }
      if (!PRE && p.x != nullptr) z[it] = add4(z[it], load_pair2<DT>(p.x, base + c));
      s += (z[it].x + z[it].y) + (z[it].z + z[it].w);
    }
  }
  const float mean = p.rms ? 0.f : wave_sum(s) * p.inv_c;  // an RMSNorm subtracts none
  float q = 0.f;
#pragma unroll
  for (int it = 0; it < ITS; ++it) {
    const int64_t c = lane + 64 * it;
    if (c < C2) {
      const float a = z[it].x - mean, b = z[it].y - mean, d = z[it].z - mean, e = z[it].w - mean;
      q += (a * a + b * b) + (d * d + e * e);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * p.inv_c + p.eps);
#pragma unroll
  for (int it = 0; it < ITS; ++it) {
    const int64_t c = lane + 64 * it;
    if (c < C2) {
      const float4 g = reinterpret_cast<const float4*>(p.gamma)[c];
      const float4 bb = reinterpret_cast<const float4*>(p.beta)[c];
      float4 o = make_float4((z[it].x - mean) * rstd * g.x + bb.x, (z[it].y - mean) * rstd * g.y + bb.y,
                             (z[it].z - mean) * rstd * g.z + bb.z, (z[it].w - mean) * rstd * g.w + bb.w);
      if constexpr (PRE) o = add4(o, load_pair2<DT>(p.x, base + c));  // x + LN(y)
      store_pair2<DT>(p.out, base + c, o);
    }
  }
}

// ------------------------------------------- local branch: windowed attention
//
// The sliding-window attention branch (SPECTRE article, section 3.2's
// use_local_branch and section 4.3): for token t of head h, the keys j with
// t - WL <= j <= t + WR inside the sequence, scores (q_t . k_j) / sqrt(D),
// softmax over those keys, y_loc[t] = sum_j p_j v_j.
//
// One workgroup of four waves per (128-query block, head, batch element).
// The block's key range goes through LDS in tiles of 32 keys, each tile
// loaded once from HBM / L2 by all 256 lanes, converted to bfloat16 once and
// read by every wave whose queries' windows reach it; the next tile's loads
// are in flight while the current one is used (two LDS buffers, one barrier
// per tile).  Each wave (32 queries) makes one pass over its tiles with the
// running-max softmax.  Both products run on MFMA
// (v_mfma_f32_32x32x16_bf16, binary32 accumulation):
//   S^T (32 keys x 32 queries) = K_tile (keys x D) . Q_tile^T (D x queries):
//     lane l supplies K[key l % 32][16 kc + 8 (l / 32) + e] and
//     Q[query l % 32][the same dims], e < 8, for the D / 16 chunks kc;
//     lane l receives the scores of query l % 32 for the keys
//     (v % 4) + 8 (v / 4) + 4 (l / 32), v < 16 -- so a query's max and sum
//     need only its own lane and lane l ^ 32;
//   O (32 queries x D) += P (queries x keys) . V (keys x D), per 32-dim tile:
//     the lane's 16 probabilities are already the A operand of the two
//     16-key chunks (the key order inside a contraction is free), so LDS
//     holds V transposed with its keys in that order (slot 16 c + 8 h + e
//     is key (e % 4) + 8 (e / 4) + 16 c + 4 h): lane l reads its dim's 8
//     keys as one 16-byte row piece.  O's element v of lane l is query
//     (v % 4) + 8 (v / 4) + 4 (l / 32), dim l % 32, so the per-query
//     rescale and the final 1 / sum reach O through 32 floats of LDS.
// Binary32 storage splits every operand into bfloat16 hi + lo (hi the
// rounded value, lo the rounded remainder: 16 significant bits) and sums the
// products hi.hi + hi.lo + lo.hi; bfloat16 storage is exact in hi, and only
// the probabilities are split.  Rows past the sequence end are clamped to
// its last row on load (every load unconditional) and masked in the scores.

// max / sum of a value over lanes l and l ^ 32 (one v_permlane32_swap:
// each half receives the other half's value)
__device__ __forceinline__ float xhalf_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

struct LocalParams {
  const void* q;
  const void* k;
  const void* v;
  float* y;        // [B][L][H][D] binary32
  int64_t L;
  int B, H, C;     // C = H * D
  int WL, WR;      // window: keys t - WL .. t + WR (each below L)
  float scale2;    // log2(e) / sqrt(D): scores in base-2 exponent units
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two binary32 values rounded to bfloat16 (one conversion), packed.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// hi = rounded pair, lo = the rounded remainders (f - hi is exact in binary32).
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// LDS image of one staged key tile, in bfloat16 elements: PL planes (hi,
// and lo for binary32 storage) of K [32 keys][KS] and of V^T [D dims][VS].
// The row strides (16 bytes of padding) make the 16-byte reads of 8
// consecutive lanes fall on distinct banks; in V^T row d the four 8-slot
// blocks are rotated by (d / 8) % 4 blocks, which spreads the staging
// writes of 16 dims that share a slot over the banks (8-way conflicts
// without it).
template <int DT, int D>
struct LocalLds {
  static constexpr int PL = DT != IN_BF16 ? 2 : 1;
  static constexpr int KS = D + 8;
  static constexpr int VS = 40;
  static constexpr int KPL = 32 * KS;
  static constexpr int VPL = D * VS;
  static constexpr int TILE = PL * (KPL + VPL);
  static constexpr int UNITS = 4 * D;  // staging units per tensor and tile
  // element offset of V^T slot `slot` (16 c + 8 h + e) in dim row `dim`
  __device__ static constexpr int vslot(int dim, int slot) {
    return dim * VS + ((slot + 8 * (dim >> 3)) & 31);
  }
};

// One thread's share of a tile in flight, as raw words: K units of 8
// consecutive dims of one key, V units of 4 consecutive dims of two keys
// that are neighbours in the V^T slot order.  NT threads stage a tile;
// units past the last repeat the last one (every load unconditional, so
// the wait before a store counts only older loads).
template <int DT, int D, int NT>
struct LocalStage {
  using LL = LocalLds<DT, D>;
  static constexpr bool F32 = DT != IN_BF16;
  static constexpr int KW = F32 ? 2 : 1;  // 16-byte words per K unit
  static constexpr int UPT = (LL::UNITS + NT - 1) / NT;
  uint4 kw[UPT][KW];
  uint4 vw[UPT][2];  // rows key, key + 1 (bfloat16: .x, .y used)

  // kt, vt: bytes of (key j0, dim 0) of this head; keys j0 + r, r > lim,
  // read row j0 + lim
  __device__ __forceinline__ void load(const char* kt, const char* vt, int lim, int C, int tid) {
    constexpr uint32_t es = F32 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      int u = tid + NT * i;
      u = u < LL::UNITS ? u : LL::UNITS - 1;
      {
        const int key = u / (D / 8), c8 = u % (D / 8);
        const uint32_t o = (__umul24((uint32_t)(key < lim ? key : lim), (uint32_t)C) + 8 * c8) * es;
#pragma unroll
        for (int x = 0; x < KW; ++x) kw[i][x] = *reinterpret_cast<const uint4*>(kt + o + 16 * x);
      }
      {
        const int kp = u / (D / 4), quad = u % (D / 4);
        const int pos = 2 * kp;  // slot 16 c + 8 h + e, e even
        const int key = (pos & 3) + 8 * ((pos >> 2) & 1) + 16 * (pos >> 4) + 4 * ((pos >> 3) & 1);
        const int k0 = key < lim ? key : lim, k1 = key + 1 < lim ? key + 1 : lim;
        const uint32_t o0 = (__umul24((uint32_t)k0, (uint32_t)C) + 4 * quad) * es;
        const uint32_t o1 = (__umul24((uint32_t)k1, (uint32_t)C) + 4 * quad) * es;
        if constexpr (F32) {
          vw[i][0] = *reinterpret_cast<const uint4*>(vt + o0);
          vw[i][1] = *reinterpret_cast<const uint4*>(vt + o1);
        } else {
          const uint2 a = *reinterpret_cast<const uint2*>(vt + o0);
          const uint2 c = *reinterpret_cast<const uint2*>(vt + o1);
          vw[i][0] = make_uint4(a.x, a.y, 0u, 0u);
          vw[i][1] = make_uint4(c.x, c.y, 0u, 0u);
        }
      }
    }
  }

  // 8 dims of a row, split (binary32 storage) or copied, into planes at d
  __device__ static void put_row8(uint16_t* d, uint4 a, uint4 c) {
    if constexpr (F32) {
      uint4 h, l;
      split_pair(__uint_as_float(a.x), __uint_as_float(a.y), h.x, l.x);
      split_pair(__uint_as_float(a.z), __uint_as_float(a.w), h.y, l.y);
      split_pair(__uint_as_float(c.x), __uint_as_float(c.y), h.z, l.z);
      split_pair(__uint_as_float(c.z), __uint_as_float(c.w), h.w, l.w);
      *reinterpret_cast<uint4*>(d) = h;
      *reinterpret_cast<uint4*>(d + LL::KPL) = l;
    } else {
      *reinterpret_cast<uint4*>(d) = a;
    }
  }

  __device__ __forceinline__ void store(uint16_t* t, int tid) const {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      int u = tid + NT * i;
      u = u < LL::UNITS ? u : LL::UNITS - 1;
      {
        const int row = u / (D / 8), c8 = u % (D / 8);
        put_row8(t + row * LL::KS + 8 * c8, kw[i][0], kw[i][KW - 1]);
      }
      {
        const int kp = u / (D / 4), quad = u % (D / 4);
        // the 4 dims share one 8-dim group, so one rotated slot for all
        uint16_t* vd = t + LL::PL * LL::KPL + LL::vslot(4 * quad, 2 * kp);
        const uint4 a = vw[i][0], c = vw[i][1];
        if constexpr (F32) {
          const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            uint32_t h, l;
            split_pair(__uint_as_float(aw[d]), __uint_as_float(cw[d]), h, l);
            *reinterpret_cast<uint32_t*>(vd + d * LL::VS) = h;
            *reinterpret_cast<uint32_t*>(vd + d * LL::VS + LL::VPL) = l;
          }
        } else {
          // dims 4 quad + d of keys key, key + 1: low / high halves of the words
          *reinterpret_cast<uint32_t*>(vd) = (a.x & 0xffffu) | (c.x << 16);
          *reinterpret_cast<uint32_t*>(vd + LL::VS) = (a.x >> 16) | (c.x & 0xffff0000u);
          *reinterpret_cast<uint32_t*>(vd + 2 * LL::VS) = (a.y & 0xffffu) | (c.y << 16);
          *reinterpret_cast<uint32_t*>(vd + 3 * LL::VS) = (a.y >> 16) | (c.y & 0xffff0000u);
        }
      }
    }
  }
};

// One wave's 32 queries: their Q operands, running max and sum, and O.
template <int DT, int D>
struct LocalWave {
  using LL = LocalLds<DT, D>;
  using E = typename std::conditional<DT != IN_BF16, float, uint16_t>::type;
  static constexpr bool F32 = DT != IN_BF16;
  static constexpr int KC = D / 16;
  static constexpr int DTL = (D + 31) / 32;
  static constexpr float NEG = -1e30f;  // max before any key: exp2 of masked scores stays 0
  bf16x8_t qh[KC], ql[KC];
  float m, lsum;
  f32x16_t o[DTL];

  __device__ void reset() {
    m = NEG;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < DTL; ++dt) o[dt] = f32x16_t{};
  }

  // Q^T operand from global memory: qr = this lane's row at dim 8 half
  __device__ void q_global(const E* qr) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if constexpr (F32) {
        const float4 a = *reinterpret_cast<const float4*>(qr + 16 * kc);
        const float4 c = *reinterpret_cast<const float4*>(qr + 16 * kc + 4);
        uint4 hh, ll;
        split_pair(a.x, a.y, hh.x, ll.x);
        split_pair(a.z, a.w, hh.y, ll.y);
        split_pair(c.x, c.y, hh.z, ll.z);
        split_pair(c.z, c.w, hh.w, ll.w);
        qh[kc] = __builtin_bit_cast(bf16x8_t, hh);
        ql[kc] = __builtin_bit_cast(bf16x8_t, ll);
      } else {
        qh[kc] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qr + 16 * kc));
      }
    }
  }

  // One staged key tile t.  Element v of the lane's scores is key
  // (v % 4) + 8 (v / 4) of the tile's keys plus 4 half; it is in the query's
  // window iff (dn + (v % 4) + 8 (v / 4)) <= qwin as unsigned numbers (the
  // caller offsets dn so that the window starts at 0).  bw: this wave's 32
  // floats of LDS.
  __device__ void step(const uint16_t* t, int dn, uint32_t qwin, float scale2, float* bw, int half,
                       int c32) {
    // scores
    f32x16_t acc = {};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint16_t* kr = t + c32 * LL::KS + 16 * kc + 8 * half;
      const bf16x8_t kh = *reinterpret_cast<const bf16x8_t*>(kr);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[kc], acc, 0, 0, 0);
      if constexpr (F32) {
        const bf16x8_t kl = *reinterpret_cast<const bf16x8_t*>(kr + LL::KPL);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, ql[kc], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qh[kc], acc, 0, 0, 0);
      }
    }
    // mask, tile max
    float s[16];
    float tmax = NEG;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int d = dn + (v & 3) + 8 * (v >> 2);
      s[v] = (uint32_t)d <= qwin ? acc[v] : -INFINITY;
      tmax = fmaxf(tmax, s[v]);
    }
    tmax = xhalf_max(tmax) * scale2;  // both halves of the query, scaled (scale2 > 0)
    // The reference max m moves only when a score exceeds it by more than
    // 2^8 (so p <= 256): O and the sum are rescaled on those tiles only, and
    // the result, O / sum, does not depend on which m was used.
    const bool up = tmax > m + 8.0f;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      const float alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.0f;
      m = up ? tmax : m;
      lsum *= alpha;
      // O's queries' alpha through this wave's own LDS slots (the wave's LDS
      // accesses run in order, so no barrier)
      if (half == 0) bw[c32] = alpha;
      __builtin_amdgcn_wave_barrier();
      float4 a4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) a4[g] = reinterpret_cast<const float4*>(bw)[2 * g + half];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int dt = 0; dt < DTL; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          o[dt][4 * g + 0] *= a4[g].x;
          o[dt][4 * g + 1] *= a4[g].y;
          o[dt][4 * g + 2] *= a4[g].z;
          o[dt][4 * g + 3] *= a4[g].w;
        }
    }
    float ps = 0.f;
    bf16x8_t ph[2], pl[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t hp[4], lp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * c + 2 * i], scale2, -m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * c + 2 * i + 1], scale2, -m));
        ps += p0 + p1;
        split_pair(p0, p1, hp[i], lp[i]);
      }
      ph[c] = __builtin_bit_cast(bf16x8_t, make_uint4(hp[0], hp[1], hp[2], hp[3]));
      pl[c] = __builtin_bit_cast(bf16x8_t, make_uint4(lp[0], lp[1], lp[2], lp[3]));
    }
    lsum += ps;
    // O += P V
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < DTL; ++dt) {
        const int dim = 32 * dt + c32;
        bf16x8_t vh = {}, vl = {};
        const uint16_t* vr = t + LL::PL * LL::KPL + LL::vslot(dim < D ? dim : 0, 16 * c + 8 * half);
        if (D % 32 == 0 || dim < D) {
          vh = *reinterpret_cast<const bf16x8_t*>(vr);
          if constexpr (F32) vl = *reinterpret_cast<const bf16x8_t*>(vr + LL::VPL);
        }
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[c], vh, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl[c], vh, o[dt], 0, 0, 0);
        if constexpr (F32) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[c], vl, o[dt], 0, 0, 0);
      }
  }

  // O / sum into y: yt = row of the wave's first query (dim 0 of the head),
  // nq of its 32 queries inside the sequence.
  __device__ void finish(float* yt, int nq, int C, float* bw, int half, int c32) {
    const float lt = xhalf_sum(lsum);  // both halves' partial sums
    if (half == 0) bw[c32] = lt > 0.f ? 1.0f / lt : 0.f;
    __builtin_amdgcn_wave_barrier();
    float4 r4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) r4[g] = reinterpret_cast<const float4*>(bw)[2 * g + half];
    __builtin_amdgcn_wave_barrier();
    // O element v of lane (dim 32 dt + c32, half): query (v % 4) + 8 (v / 4) + 4 half.
    // Addresses: a wave-uniform row pointer per (g, i) plus one per-lane
    // byte offset, so no per-store 64-bit offsets stay live.
    const uint32_t laneoff = (__umul24(4u * half, (uint32_t)C) + c32) * 4u;
    auto store = [&](bool full) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float rg[4] = {r4[g].x, r4[g].y, r4[g].z, r4[g].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const char* rowp = reinterpret_cast<const char*>(yt) + (size_t)(i + 8 * g) * C * 4;
          if (!full && i + 8 * g + 4 * half >= nq) continue;
#pragma unroll
          for (int dt = 0; dt < DTL; ++dt) {
            if (D % 32 != 0 && 32 * dt + c32 >= D) continue;
            *reinterpret_cast<float*>(const_cast<char*>(rowp) + laneoff + 128 * dt) = o[dt][4 * g + i] * rg[i];
          }
        }
      }
    };
    if (nq == 32)
      store(true);  // every query of the wave is in the sequence: no per-row test
    else
      store(false);
  }
};

// One workgroup of four waves per (128-query block, head, batch element);
// the block's key range streams through LDS once.
template <int DT, int D>
__device__ __forceinline__ void local_block(const LocalParams& p) {
  using LL = LocalLds<DT, D>;
  using E = typename std::conditional<DT != IN_BF16, float, uint16_t>::type;
  using Stage = LocalStage<DT, D, 256>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * LL::TILE];
  __shared__ float4 bc[4][8];  // per wave: 32 per-query factors, broadcast to O's layout
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave: uniform
  const int half = lane >> 5, c32 = lane & 31;
  const int C = p.C;
  // work item: 128-query block fastest, then head, then batch element; the
  // workgroups one XCD runs (every 8th) take a contiguous run of items, so
  // the overlapping key ranges of neighbouring blocks meet in one L2
  const int nblk = (int)((p.L + 127) / 128);
  const int nitem = nblk * p.H * p.B;
  int w = blockIdx.x;
  if (nitem % 8 == 0) w = (w % 8) * (nitem / 8) + w / 8;
  const int blk = w % nblk;
  const int64_t T0 = (int64_t)blk * 128;
  const int h = (w / nblk) % p.H;
  const int b = w / (nblk * p.H);
  const int64_t base = (int64_t)b * p.L * C + (int64_t)h * D;  // element (b, t = 0, h, 0)
  const int64_t Lm1 = p.L - 1;
  const char* kp = reinterpret_cast<const char*>(reinterpret_cast<const E*>(p.k) + base);
  const char* vp = reinterpret_cast<const char*>(reinterpret_cast<const E*>(p.v) + base);

  // the block's keys, in tiles of 32 from jlo
  const int64_t jlo = T0 - p.WL < 0 ? 0 : T0 - p.WL;
  const int64_t jend = T0 + 127 + p.WR < Lm1 ? T0 + 127 + p.WR : Lm1;
  const int nt = (int)((jend - jlo + 32) / 32);
  auto stage_load = [&](Stage& st, int n) __attribute__((always_inline)) {
    const int j0 = (int)jlo + 32 * n;
    const int lim = (int)(Lm1 - j0 < 31 ? Lm1 - j0 : 31);
    const int64_t o = (int64_t)j0 * C * (int64_t)sizeof(E);
    st.load(kp + o, vp + o, lim, C, tid);
  };

  // this wave's 32 queries and the keys their windows reach
  const int64_t Tw = T0 + 32 * wave;
  const bool wave_on = Tw < p.L;
  const int64_t wlo = Tw - p.WL < 0 ? 0 : Tw - p.WL;
  const int64_t whi = Tw + 31 + p.WR < Lm1 ? Tw + 31 + p.WR : Lm1;
  const int64_t tq = Tw + c32;  // this lane's query (clamped on load; not stored past L)
  LocalWave<DT, D> W;
  W.reset();
  W.q_global(reinterpret_cast<const E*>(p.q) + base + (tq < Lm1 ? tq : Lm1) * C + 8 * half);
  // key j is in this lane's query window iff 0 <= j - tq + WL <= qwin
  // (for a clamped query tq >= L the test admits any key: its row is not stored)
  const uint32_t qwin = (uint32_t)((tq + p.WR < Lm1 ? tq + p.WR : Lm1) - tq + p.WL);
  const int d0 = (int)(jlo - tq + p.WL) + 4 * half;  // key (v%4)+8(v/4) of tile 0, relative
  float* bw = reinterpret_cast<float*>(bc[wave]);

  // Tile n + 1's loads go out at the start of iteration n and reach the
  // other LDS buffer at its end, after the arithmetic on tile n.  Loads and
  // stores are unconditional (the tile index clamped to the last tile; a
  // store past the last tile fills a buffer nobody reads again), so the
  // wait before each store counts only that set.
  // Even blocks start their walk 4 tiles in (one block's length): block b's
  // tile 4 + s is block b + 1's tile s, so at window 128 (8 tiles) the two
  // blocks that share a tile read it at the same step, once from HBM, and
  // likewise for block b - 1 (the softmax does not depend on the order).
  const int rot = (blk & 1) ? 0 : 4 % nt;
  auto tile_of = [&](int n) { return n + rot < nt ? n + rot : n + rot - nt; };
  Stage st;
  stage_load(st, tile_of(0));
  st.store(lds, tid);
  __syncthreads();
#pragma unroll 1
  for (int n = 0; n < nt; ++n) {
    stage_load(st, tile_of(n + 1 < nt ? n + 1 : nt - 1));
    const int tn = tile_of(n);
    const int64_t k0 = jlo + 32 * tn;
    if (wave_on && k0 <= whi && k0 + 31 >= wlo)
      W.step(lds + (n & 1) * LL::TILE, d0 + 32 * tn, qwin, p.scale2, bw, half, c32);
    st.store(lds + ((n + 1) & 1) * LL::TILE, tid);
    __syncthreads();
  }
  if (!wave_on) return;
  W.finish(p.y + base + Tw * C, (int)(p.L - Tw < 32 ? p.L - Tw : 32), C, bw, half, c32);
}

// Head sizes up to 64 fit three workgroups per CU in registers and LDS
// (four with bfloat16 storage, which needs no split of K and V); 128 takes
// what its registers allow.
template <int DT, int D>
__global__ __launch_bounds__(256, DT == IN_BF16 ? 4 : 3) void k_local_attn(LocalParams p) {
  local_block<DT, D>(p);
}

template <int DT>
__global__ __launch_bounds__(256) void k_local_attn_wide(LocalParams p) {
  local_block<DT, 128>(p);
}

// Chunked mix, y only, single-level blocks: y[b][t][pair] += yblk[b][pair]
// over nb blocks of Lb tokens (b = the block).
__global__ __launch_bounds__(256) void k_block_add(float2* y, const float2* yblk, int64_t n,
                                                   int64_t Lb, int64_t CP2) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = cadd(y[i], yblk[(i / (Lb * CP2)) * CP2 + i % CP2]);
}

}  // namespace spectre
