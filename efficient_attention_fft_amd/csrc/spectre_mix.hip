// spectre_mix.hip -- host side of the SPECTRE spectral-mix library (C ABI).
//
// Validates arguments (before any device call), plans the transform of
// length L, keeps per-device twiddle tables and a workspace, and enqueues
// the gfx950 kernels of kernels.hpp on the caller's stream.  The operation is
// the one the SPECTRE FFT-attention article describes in section 2.2 (with
// section 2.3's truncation); the C ABI and its conventions are documented in
// include/spectre_mix.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/spectre_mix.h"
#include "kernels.hpp"

namespace spectre {
namespace {

// ------------------------------------------------------------------ plan

constexpr int64_t kMaxL = 3 * (int64_t(1) << 20);
constexpr int64_t kMaxSingle = 2048;  // longest length for the single-level k_mid / k_mid_sq
                                      // (3072 and 4096 have the column kernel k_col)
constexpr int kMaxC = 4096;
constexpr int kMaxMidThreads = 512;   // launch bound of the B kernel
constexpr int kMaxFusedPairs = 256; // launch bound of the fused C1 kernel
constexpr int kLdsBudget = 64 * 1024;  // bytes of LDS per B workgroup

struct Plan {
  int64_t L = 0, L1 = 1, L2 = 1, L3 = 1;
  int col = 0;  // single-level plan run by the column kernel k_col: its ColKind, else 0
  int sq = 0;  // R when L3 = R * R uses the two-register-DFT B kernel (R = 16, 32), else 0
  int P = 0;   // points per thread in B
  int Tc = 0;  // threads per column in B
  int nrad = 0;
  int rad[8] = {0};
};

// 2^a * 3^b decomposition; false if L has another prime factor.
bool factor23(int64_t L, int& a, int& b) {
  a = b = 0;
  while (L > 1 && L % 2 == 0) {
    L /= 2;
    ++a;
  }
  while (L > 1 && L % 3 == 0) {
    L /= 3;
    ++b;
  }
  return L == 1;
}

bool strided_size_ok(int64_t r) {
  switch (r) {
    case 2: case 3: case 4: case 6: case 8: case 12: case 16: case 24: case 32: case 48: case 64:
      return true;
    default:
      return false;
  }
}

// Radices (each dividing P) whose product is N, largest first.
bool plan_radices(int64_t N, int P, Plan& pl) {
  static const int cand[] = {16, 12, 8, 6, 4, 3, 2};
  pl.nrad = 0;
  int64_t rem = N;
  while (rem > 1) {
    int pick = 0;
    for (int r : cand)
      if (P % r == 0 && rem % r == 0) {
        pick = r;
        break;
      }
    if (!pick || pl.nrad == 8) return false;
    pl.rad[pl.nrad++] = pick;
    rem /= pick;
  }
  return true;
}

// Lengths the single-pass column kernel runs, L = RA * RB * RC (ColCfg).  At
// 6144 and 8192 its first stage (24 or 32 points per thread) needs more
// registers than four waves per SIMD leave, and the four-step plan is faster.
enum ColKind { COL_NONE = 0, COL_3072 = 1, COL_4096 = 2 };

int col_kind(int64_t L) {
  switch (L) {
    case 3072: return COL_3072;
    case 4096: return COL_4096;
    default: return COL_NONE;
  }
}

// The column kernel runs one workgroup per 4 channel pairs of a batch
// element, one per CU, and its transform, LDS exchanges and memory phases do
// not overlap inside a CU; it beats the four-step plan (whose last pass also
// fuses the norm) only while its whole grid is one round on the chip's 256
// CUs.  Larger calls at these lengths take the four-step plan.
constexpr int64_t kColMaxItems = 256;

bool col_fits(int64_t B, int64_t CP2) { return B * ((CP2 + 3) / 4) <= kColMaxItems; }

int make_plan(int64_t L, Plan& pl, bool allow_col = true) {
  pl = Plan();
  if (L < 2 || L % 2 != 0) return SPECTRE_EINVAL;
  int a = 0, b = 0;
  if (!factor23(L, a, b) || b > 1 || L > kMaxL) return SPECTRE_EUNSUPPORTED;
  pl.L = L;
  if (int ck = allow_col ? col_kind(L) : COL_NONE) {  // one pass: the whole column in LDS
    pl.L3 = L;
    pl.col = ck;
    return SPECTRE_OK;
  }
  if (L <= kMaxSingle) {
    pl.L3 = L;
  } else {
    // L3: power of two <= 1024, leaving at least one factor 2 for an even L1
    int64_t l3 = int64_t(1) << std::min(a - 1, 10);
    int64_t rest = L / l3;
    int64_t l1 = rest, l2 = 1;
    if (rest > 64) {
      int a_rest = a - (int)std::log2((double)l3);
      l1 = int64_t(1) << std::min(a_rest, 6);
      l2 = rest / l1;
    }
    if (l1 % 2 != 0 || !strided_size_ok(l1) || (l2 != 1 && !strided_size_ok(l2)))
      return SPECTRE_EUNSUPPORTED;
    pl.L1 = l1;
    pl.L2 = l2;
    pl.L3 = l3;
  }
  const int64_t N = pl.L3;
  if (N % 3 == 0)
    pl.P = N >= 12 ? 12 : 6;
  else
    pl.P = (int)std::min<int64_t>(16, N);
  pl.Tc = (int)(N / pl.P);
  if (!plan_radices(N, pl.P, pl)) return SPECTRE_EUNSUPPORTED;
  if (N == 1024) pl.sq = 32;
  if (N == 256) pl.sq = 16;
  return SPECTRE_OK;
}

bool is_single(const Plan& pl) { return pl.L1 == 1 && pl.L2 == 1; }

// Channel pairs per workgroup slot in B: a power of two dividing CP2, with
// the thread count and the LDS tile inside their budgets.
int choose_cpt(const Plan& pl, int64_t CP2, int nslot) {
  int cpt = 1;
  while (true) {
    int next = cpt * 2;
    if (CP2 % next != 0) break;
    if ((int64_t)pl.Tc * nslot * next > kMaxMidThreads) break;
    if (pl.L3 * nslot * next * 8 > kLdsBudget) break;
    if (next > 16) break;
    cpt = next;
  }
  return cpt;
}

// Channel pairs per slot for the square B kernel: 256 threads when possible.
int choose_cpt_sq(int R, int64_t CP2, int nslot) {
  int cpt = 256 / (R * nslot);
  while (cpt > 1 && CP2 % cpt != 0) cpt /= 2;
  return cpt;
}

// Whether C1 can hold every channel of a token in one workgroup.
bool fused_norm_ok(int64_t CP2) { return CP2 % 64 == 0 && CP2 <= kMaxFusedPairs; }

// ----------------------------------------------------------- tables cache

struct LenTables {
  float2* twL = nullptr;   // L entries
  float2* twN = nullptr;   // L3 entries
  int2* wgcols = nullptr;  // column workgroups of B
  int nwg = 0;
  int selfwg = -1;
};

struct DeviceState {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::map<int64_t, LenTables> tables;  // keyed by table_key(plan)
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;

// Per-device facts kept in fixed arrays (no allocation on any path).
constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices] = {0};  // compute units, queried once; guarded by g_mu

int cu_count(int dev, int* cus) {
  if (dev < 0 || dev >= kMaxDevices) return SPECTRE_EUNSUPPORTED;
  if (g_cus[dev] <= 0 &&
      (hipDeviceGetAttribute(&g_cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
       g_cus[dev] <= 0))
    return SPECTRE_EHIP;
  *cus = g_cus[dev];
  return SPECTRE_OK;
}

// Dynamic LDS above 64 KB needs the kernel's attribute raised, once per
// (function, device); `done` holds one bit per device already set.
int lds_attr(const void* fn, int bytes, uint64_t& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPECTRE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SPECTRE_EUNSUPPORTED;
  const uint64_t bit = uint64_t(1) << dev;
  if (done & bit) return SPECTRE_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    return SPECTRE_EHIP;
  done |= bit;
  return SPECTRE_OK;
}

// ---------------------------------------------------------------- tracing
//
// Optional per-kernel HIP events: one before a traced call's first kernel,
// one after each kernel.  Guarded by g_mu like everything else.

constexpr int kMaxKernelsPerCall = 8;

struct TraceCall {
  size_t first = 0;  // index of the call's first event in the pool
  int nk = 0;
  const char* names[kMaxKernelsPerCall] = {nullptr};
};

struct TraceState {
  bool on = false;
  int max_calls = 0;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<TraceCall> calls;
  bool active = false;  // the current call is being traced
  hipStream_t stream = nullptr;
};

TraceState g_trace;

void trace_call_begin(hipStream_t st) {
  g_trace.active = false;
  if (!g_trace.on || (int)g_trace.calls.size() >= g_trace.max_calls) return;
  if (g_trace.used + kMaxKernelsPerCall + 1 > g_trace.pool.size()) return;
  TraceCall c;
  c.first = g_trace.used;
  if (hipEventRecord(g_trace.pool[g_trace.used], st) != hipSuccess) return;
  ++g_trace.used;
  g_trace.calls.push_back(c);
  g_trace.active = true;
  g_trace.stream = st;
}

void trace_kernel(const char* name) {
  if (!g_trace.active) return;
  TraceCall& c = g_trace.calls.back();
  if (c.nk >= kMaxKernelsPerCall) return;
  if (hipEventRecord(g_trace.pool[g_trace.used], g_trace.stream) != hipSuccess) return;
  ++g_trace.used;
  c.names[c.nk++] = name;
}

// Renames the current call's last traced kernel (a pass launched through a
// shared launcher for another role).
void trace_rename_last(const char* name) {
  if (!g_trace.active) return;
  TraceCall& c = g_trace.calls.back();
  if (c.nk > 0) c.names[c.nk - 1] = name;
}

// exp(-2 pi i e / n) in double, angle split exactly into a quarter turn and
// a residual of at most pi/4, then rounded to binary32 (host tables, and the
// allocation-free entry point's table kernel).
__host__ __device__ float2 host_twiddle(int64_t e, int64_t n) {
  constexpr double kHalfPi = 1.57079632679489661923;
  e %= n;
  int64_t q = (4 * e + n / 2) / n;
  int64_t r = 4 * e - q * n;
  double phi = kHalfPi * (double)r / (double)n;
  double c = cos(phi), s = sin(phi);
  double re, im;
  switch (q & 3) {
    case 0: re = c; im = s; break;
    case 1: re = -s; im = c; break;
    case 2: re = -c; im = -s; break;
    default: re = s; im = -c; break;
  }
  return make_float2((float)re, (float)-im);
}

// Column workgroups of B: each regular workgroup holds a column and its
// mirror column; the two self-paired columns share one workgroup, column
// (0, 0) in slot 0.  Single-level plans have one column per batch.
void build_wgcols(const Plan& pl, std::vector<int2>& out, int& selfwg) {
  out.clear();
  selfwg = -1;
  if (is_single(pl)) {
    out.push_back(make_int2(0, -1));
    return;
  }
  const int64_t L1 = pl.L1, L2 = pl.L2;
  std::vector<int> self;
  for (int64_t k2 = 0; k2 < L2; ++k2)
    for (int64_t k1 = 0; k1 < L1; ++k1) {
      int64_t pk1, pk2;
      if (k1 != 0) {
        pk1 = L1 - k1;
        pk2 = L2 - 1 - k2;
      } else {
        pk1 = 0;
        pk2 = (L2 - k2) % L2;
      }
      int64_t c = k1 + L1 * k2, pc = pk1 + L1 * pk2;
      if (c == pc)
        self.push_back((int)c);
      else if (c < pc)
        out.push_back(make_int2((int)c, (int)pc));
    }
  // column (0, 0) first: its mirror map is k3 -> (N - k3) mod N
  int2 s = make_int2(-1, -1);
  if (!self.empty()) s.x = self[0];
  if (self.size() > 1) s.y = self[1];
  selfwg = (int)out.size();
  out.push_back(s);
}

// Tables are cached per (device, plan): one length can have two plans (the
// column kernel's single pass and the four-step), whose tables differ.
int64_t table_key(const Plan& pl) { return pl.L * 2 + (pl.col ? 1 : 0); }

int get_tables(int dev, const Plan& pl, LenTables** res) {
  DeviceState& ds = g_dev[dev];
  auto it = ds.tables.find(table_key(pl));
  if (it != ds.tables.end()) {
    *res = &it->second;
    return SPECTRE_OK;
  }
  LenTables t;
  std::vector<float2> twL(pl.L), twN(pl.L3);
  for (int64_t e = 0; e < pl.L; ++e) twL[e] = host_twiddle(e, pl.L);
  for (int64_t e = 0; e < pl.L3; ++e) twN[e] = host_twiddle(e, pl.L3);
  std::vector<int2> cols;
  build_wgcols(pl, cols, t.selfwg);
  t.nwg = (int)cols.size();
  if (hipMalloc(&t.twL, sizeof(float2) * pl.L) != hipSuccess) return SPECTRE_ENOMEM;
  if (hipMalloc(&t.twN, sizeof(float2) * pl.L3) != hipSuccess ||
      hipMalloc(&t.wgcols, sizeof(int2) * cols.size()) != hipSuccess) {
    (void)hipFree(t.twL);
    (void)hipFree(t.twN);
    return SPECTRE_ENOMEM;
  }
  if (hipMemcpy(t.twL, twL.data(), sizeof(float2) * pl.L, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(t.twN, twN.data(), sizeof(float2) * pl.L3, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(t.wgcols, cols.data(), sizeof(int2) * cols.size(), hipMemcpyHostToDevice) !=
          hipSuccess) {
    (void)hipFree(t.twL);
    (void)hipFree(t.twN);
    (void)hipFree(t.wgcols);
    return SPECTRE_EHIP;
  }
  auto ins = ds.tables.emplace(table_key(pl), t);
  *res = &ins.first->second;
  return SPECTRE_OK;
}

bool fail_alloc_forced() {
  const char* e = std::getenv("SPECTRE_MIX_FAIL_ALLOC");
  return e && e[0] == '1';
}

int get_workspace(int dev, size_t bytes, void** ws) {
  DeviceState& ds = g_dev[dev];
  if (fail_alloc_forced()) return SPECTRE_ENOMEM;
  if (ds.ws_bytes < bytes) {
    if (ds.ws) {
      // the previous workspace may still be in use by enqueued work
      if (hipDeviceSynchronize() != hipSuccess) return SPECTRE_EHIP;
      (void)hipFree(ds.ws);
      ds.ws = nullptr;
      ds.ws_bytes = 0;
    }
    if (hipMalloc(&ds.ws, bytes) != hipSuccess) {
      ds.ws = nullptr;
      return SPECTRE_ENOMEM;
    }
    ds.ws_bytes = bytes;
  }
  *ws = ds.ws;
  return SPECTRE_OK;
}

// ------------------------------------------------------------ validation

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

struct Shape {
  int64_t B, H, L, D, C, CP2, N;
  int64_t keep;
  int dtype;
  size_t esz;
  int gate_kind;   // spectre_gate_kind
  int norm_order;  // spectre_norm_order
};

// Chunked mix (blocks of L tokens of the blockwise shape, nb per batch
// element): the block-axis step's gate and kept bins.
struct Chunk {
  const float* gate_blocks;  // [H][nb/2 + 1]
  int64_t nb;                // blocks per batch element
  int64_t keep_blocks;
  int64_t B;                 // batch elements (the blockwise shape has B * nb)
};

// Local branch: keys t - wl .. t + wr of token t (clipped to the sequence).
struct Local {
  int64_t wl, wr;
  const float* mix;  // per-channel gate of the two branches, or null (summed)
};

int check_shape(int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep, int dtype, Shape& s,
                Plan& pl, int gate_kind = SPECTRE_GATE_REAL, int norm_order = SPECTRE_NORM_POST) {
  if (B < 1 || H < 1 || D < 1 || L < 2) return SPECTRE_EINVAL;
  if (dtype != SPECTRE_F32 && dtype != SPECTRE_BF16) return SPECTRE_EINVAL;
  if (gate_kind != SPECTRE_GATE_REAL && gate_kind != SPECTRE_GATE_LOGIT &&
      gate_kind != SPECTRE_GATE_COMPLEX)
    return SPECTRE_EINVAL;
  if (norm_order < SPECTRE_NORM_POST || norm_order > SPECTRE_NORM_PRE_RMS) return SPECTRE_EINVAL;
  if (L % 2 != 0) return SPECTRE_EINVAL;
  if (keep < 0 || keep > L / 2 + 1) return SPECTRE_EINVAL;
  if (H > kMaxC || D > kMaxC || H * D > kMaxC) return SPECTRE_EUNSUPPORTED;
  const int64_t C = H * D;
  if (C % 2 != 0) return SPECTRE_EUNSUPPORTED;
  if (L * C >= (int64_t(1) << 29)) return SPECTRE_EUNSUPPORTED;  // 32-bit byte offsets per batch
  if (B > (int64_t(1) << 40) / (L * C)) return SPECTRE_EUNSUPPORTED;
  int st = make_plan(L, pl, col_fits(B, C / 2));
  if (st != SPECTRE_OK) return st;
  s.B = B;
  s.H = H;
  s.L = L;
  s.D = D;
  s.C = C;
  s.CP2 = C / 2;
  s.N = B * L * C;
  s.keep = keep;
  s.dtype = dtype;
  s.esz = dtype == SPECTRE_F32 ? 4 : 2;
  s.gate_kind = gate_kind;
  s.norm_order = norm_order;
  return SPECTRE_OK;
}

// Two-level plans with the square B kernel hand it the spectra in the tiled
// layout ([b][k1][CP2/4][L3][4]); B then writes U (row layout) to a fourth
// region instead of in place.
bool tiled_plan(const Shape& s, const Plan& pl) {
  return !is_single(pl) && pl.L2 == 1 && pl.sq == 32 && s.CP2 % 32 == 0 && pl.L3 % 16 == 0;
}

// Three-level plans whose B is the square kernel: the second pass runs out of
// place and writes the tiled layout into three more regions; B then writes U
// over the first pass's q region.
bool tiled3_plan(const Shape& s, const Plan& pl) {
  return !is_single(pl) && pl.L2 > 1 && pl.L2 <= 32 && pl.sq == 32 && s.CP2 % 16 == 0 &&
         pl.L3 % 16 == 0;
}

// Bytes of the spectra part of the workspace: three complex spectra of pairs
// (q, k, v; U and y reuse them), a fourth region for U with the two-level
// tiled layout, six regions with the three-level one (the second pass out of
// place), y for the single-level LayerNorm pass.
size_t spectra_bytes(const Shape& s, const Plan& pl, bool want_fwd) {
  const size_t n = (size_t)s.N;
  if (is_single(pl)) return want_fwd ? 4 * n : 0;
  return (tiled3_plan(s, pl) ? 24 : tiled_plan(s, pl) ? 16 : 12) * n;
}

// Bytes of the gate table the square B kernel of a multi-level plan reads
// (H * L binary32 values, or pairs for a complex gate, in its own bin order),
// else 0.
size_t gate_table_bytes(const Shape& s, const Plan& pl) {
  const size_t per = s.gate_kind == SPECTRE_GATE_COMPLEX ? 8 : 4;
  return pl.sq && !is_single(pl) ? per * s.H * s.L : 0;
}

size_t workspace_for(const Shape& s, const Plan& pl, bool want_fwd) {
  const size_t a = (spectra_bytes(s, pl, want_fwd) + 255) & ~(size_t)255;
  return a + gate_table_bytes(s, pl);
}

// Extra workspace of a chunked mix, after the rest (256-byte aligned): the
// block means of q, k, v and the block term, 4 x B x CP2 pairs of the
// blockwise shape (one row of pairs per block).
size_t chunk_bytes(const Shape& s, const Chunk* ch) {
  return ch ? 256 + 4 * (size_t)s.B * s.CP2 * sizeof(float2) : 0;
}

// ------------------------------------------------------------ launching

#define SPECTRE_LAUNCH_CHECK(name)                            \
  do {                                                        \
    if (hipGetLastError() != hipSuccess) return SPECTRE_EHIP; \
    trace_kernel(name);                                       \
  } while (0)

template <int R, int IN>
int launch_strided_fwd(const StridedParams& p, int tw, int ntensor, hipStream_t st, bool tiled) {
  const int64_t lines = p.outer * p.inner * p.CP2;
  const unsigned planes = ntensor + (p.gt.gtab ? 1 : 0);
  if (tiled) {
    const int64_t wgs = p.outer * (p.inner / 16) * (p.CP2 / 16);
    if (wgs > INT32_MAX) return SPECTRE_EUNSUPPORTED;
    if (tw == TW_A1)
      hipLaunchKernelGGL((k_strided<R, IN, TW_A1, -1, true>), dim3((unsigned)wgs, planes), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((k_strided<R, IN, TW_A2, -1, true>), dim3((unsigned)wgs, planes), dim3(256), 0, st, p);
    SPECTRE_LAUNCH_CHECK(tw == TW_A1 ? "A1_fwd_strided" : "A2_fwd_strided");
    return SPECTRE_OK;
  }
  dim3 grid((unsigned)((lines + 255) / 256), planes);
  if (tw == TW_A1)
    hipLaunchKernelGGL((k_strided<R, IN, TW_A1, -1>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_strided<R, IN, TW_A2, -1>), grid, dim3(256), 0, st, p);
  SPECTRE_LAUNCH_CHECK(tw == TW_A1 ? "A1_fwd_strided" : "A2_fwd_strided");
  return SPECTRE_OK;
}

template <int R, int IN>
int launch_strided_fwd_split(const StridedParams& p, int tw, int ntensor, bool tiled, hipStream_t st) {
  const int64_t lines = p.outer * p.inner * p.CP2;
  const int64_t waves = (lines + 31) / 32;
  dim3 grid((unsigned)((waves + 3) / 4), ntensor + (p.gt.gtab ? 1 : 0));
  if (tiled && tw == TW_A1)
    hipLaunchKernelGGL((k_strided_split<R, IN, TW_A1, true>), grid, dim3(256), 0, st, p);
  else if (tw == TW_A1)
    hipLaunchKernelGGL((k_strided_split<R, IN, TW_A1, false>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_strided_split<R, IN, TW_A2, false>), grid, dim3(256), 0, st, p);
  SPECTRE_LAUNCH_CHECK(tw == TW_A1 ? "A1_fwd_strided" : "A2_fwd_strided");
  return SPECTRE_OK;
}

// Forward strided pass of length R; `tiled` writes the tiled layout the
// square B kernel reads (the first pass of a two-level plan, or the second
// of a three-level one with R <= 32).
template <int IN>
int strided_fwd(int64_t R, const StridedParams& p, int tw, int ntensor, hipStream_t st,
                bool tiled = false) {
  switch (R) {
    case 2: return launch_strided_fwd<2, IN>(p, tw, ntensor, st, tiled);
    case 3: return launch_strided_fwd<3, IN>(p, tw, ntensor, st, tiled);
    case 4: return launch_strided_fwd<4, IN>(p, tw, ntensor, st, tiled);
    case 6: return launch_strided_fwd<6, IN>(p, tw, ntensor, st, tiled);
    case 8: return launch_strided_fwd<8, IN>(p, tw, ntensor, st, tiled);
    case 12: return launch_strided_fwd<12, IN>(p, tw, ntensor, st, tiled);
    case 16: return launch_strided_fwd<16, IN>(p, tw, ntensor, st, tiled);
    case 24: return launch_strided_fwd<24, IN>(p, tw, ntensor, st, tiled);
    case 32: return launch_strided_fwd<32, IN>(p, tw, ntensor, st, tiled);
    case 48: return launch_strided_fwd_split<48, IN>(p, tw, ntensor, tiled, st);
    case 64: return launch_strided_fwd_split<64, IN>(p, tw, ntensor, tiled, st);
    default: return SPECTRE_EUNSUPPORTED;
  }
}

template <int R>
int launch_strided_inv(const StridedParams& p, hipStream_t st) {
  const int64_t lines = p.outer * p.inner * p.CP2;
  dim3 grid((unsigned)((lines + 255) / 256), 1);
  hipLaunchKernelGGL((k_strided<R, IN_C32, TW_C2, +1>), grid, dim3(256), 0, st, p);
  SPECTRE_LAUNCH_CHECK("C2_inv_strided");
  return SPECTRE_OK;
}

int strided_inv(int64_t R, const StridedParams& p, hipStream_t st) {
  switch (R) {
    case 2: return launch_strided_inv<2>(p, st);
    case 3: return launch_strided_inv<3>(p, st);
    case 4: return launch_strided_inv<4>(p, st);
    case 6: return launch_strided_inv<6>(p, st);
    case 8: return launch_strided_inv<8>(p, st);
    case 12: return launch_strided_inv<12>(p, st);
    case 16: return launch_strided_inv<16>(p, st);
    case 24: return launch_strided_inv<24>(p, st);
    case 32: return launch_strided_inv<32>(p, st);
    case 48: return launch_strided_inv<48>(p, st);
    case 64: return launch_strided_inv<64>(p, st);
    default: return SPECTRE_EUNSUPPORTED;
  }
}

template <int P, int IN>
int launch_mid_p(const MidParams& p, dim3 grid, int threads, hipStream_t st) {
  const size_t lds = (size_t)p.N * p.nslot * p.cpt * sizeof(float2);
  hipLaunchKernelGGL((k_mid<P, IN>), grid, dim3(threads), lds, st, p);
  SPECTRE_LAUNCH_CHECK("B_mid_lds");
  return SPECTRE_OK;
}

template <int R, int IN, bool CG>
int launch_mid_sq_k(const MidParams& p, dim3 grid, hipStream_t st) {
  const int ncols = p.nslot * p.cpt;
  // real gate values in LDS when every workgroup's channel pairs lie in one head
  const bool one_head = p.D % 2 == 0 && (p.D / 2) % p.cpt == 0;
  const bool gl = IN == IN_C32 && !CG && p.gtab != nullptr && one_head;
  const size_t lds = ((size_t)R * (R * ncols + 1) + (size_t)R * R) * sizeof(float2) +
                     (gl ? (size_t)p.nslot * (R / 2 + 1) * R * sizeof(float) : 0);
  // tiled input, two slots of 4 pairs, R = 32, pairs of one head: the kernel
  // that copies its input blocks to LDS asynchronously
  if (IN == IN_C32 && p.gtab != nullptr && one_head && R == 32 && p.tiled && p.nslot == 2 &&
      p.cpt == 4) {
    // the product's bound from the truncation: every bin f = column + S (k1 +
    // 32 u) with u >= uk is truncated (f >= keep, and f stays below L - keep
    // while u <= 16 unless keep is near L/2, which keeps every u)
    const int64_t S = (int64_t)p.L1 * p.L2;
    const int64_t fmax = (S - 1) + S * (31 + 32 * 16);
    int uk = 17;
    if (p.L - fmax >= p.keep) {
      const int64_t need = (p.keep + 32 * S - 1) / (32 * S);
      uk = need <= 5 ? 5 : need <= 9 ? 9 : 17;
    }
    const void* fn = uk == 5 ? reinterpret_cast<const void*>(&k_mid_dma<CG, 5>)
                   : uk == 9 ? reinterpret_cast<const void*>(&k_mid_dma<CG, 9>)
                             : reinterpret_cast<const void*>(&k_mid_dma<CG, 17>);
    static uint64_t dma_attr[3] = {0, 0, 0};  // guarded by g_mu
    if (int rc = lds_attr(fn, 160 * 1024, dma_attr[uk == 5 ? 0 : uk == 9 ? 1 : 2])) return rc;
    MidParams q = p;
    q.gx = (int)grid.x;
    q.gy = (int)grid.y;
    q.gz = (int)grid.z;
    const int64_t ntile = (int64_t)grid.x * grid.y * grid.z;
    // When two workgroups per CU can hold every item in at most 4 rounds,
    // each workgroup takes that many items in turn (the next item's first
    // copy then runs under this item's end); the workgroups sharing output
    // lines (items 8 apart: with a grid that is a multiple of 32, the same
    // turn of workgroups on one XCD) stay close in time.  Larger grids keep
    // one item per workgroup: over more turns the sharers drift apart, and
    // the dispatcher's own order keeps them together.
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPECTRE_EHIP;
    if (int rc = cu_count(dev, &cus)) return rc;
    const int64_t slots = 2 * (int64_t)cus;
    int64_t wgs = ntile;
    if (ntile <= 4 * slots) {
      const int64_t items = (ntile + slots - 1) / slots;
      wgs = ((ntile + items - 1) / items + 31) / 32 * 32;
      if (wgs > ntile) wgs = ntile;
    }
    const size_t lds_dma = ((size_t)R * (R * ncols + 1) + (size_t)R * R) * sizeof(float2) +
                           (CG ? 0 : (size_t)p.nslot * (R / 2 + 1) * R * sizeof(float));
    if (uk == 5)
      hipLaunchKernelGGL((k_mid_dma<CG, 5>), dim3((unsigned)wgs), dim3(256), lds_dma, st, q);
    else if (uk == 9)
      hipLaunchKernelGGL((k_mid_dma<CG, 9>), dim3((unsigned)wgs), dim3(256), lds_dma, st, q);
    else
      hipLaunchKernelGGL((k_mid_dma<CG, 17>), dim3((unsigned)wgs), dim3(256), lds_dma, st, q);
    SPECTRE_LAUNCH_CHECK("B_mid_lds");
    return SPECTRE_OK;
  }
  static uint64_t attr_set[2] = {0, 0};  // guarded by g_mu
  const void* fn = gl ? reinterpret_cast<const void*>(&k_mid_sq<R, IN, true, CG>)
                      : reinterpret_cast<const void*>(&k_mid_sq<R, IN, false, CG>);
  if (int rc = lds_attr(fn, 160 * 1024, attr_set[gl])) return rc;
  if (gl)
    hipLaunchKernelGGL((k_mid_sq<R, IN, true, CG>), grid, dim3(R * ncols), lds, st, p);
  else
    hipLaunchKernelGGL((k_mid_sq<R, IN, false, CG>), grid, dim3(R * ncols), lds, st, p);
  SPECTRE_LAUNCH_CHECK("B_mid_lds");
  return SPECTRE_OK;
}

// The gate table holds complex values for a complex gate (multi-level);
// single-level kernels read the gate itself, whatever its kind.
template <int R, int IN>
int launch_mid_sq(const MidParams& p, dim3 grid, hipStream_t st) {
  if constexpr (IN == IN_C32) {
    if (p.gate_kind == GATE_COMPLEX) return launch_mid_sq_k<R, IN, true>(p, grid, st);
  }
  return launch_mid_sq_k<R, IN, false>(p, grid, st);
}

template <int IN>
int launch_mid_square(int R, const MidParams& p, dim3 grid, hipStream_t st) {
  if (R == 32) return launch_mid_sq<32, IN>(p, grid, st);
  if (R == 16) return launch_mid_sq<16, IN>(p, grid, st);
  return SPECTRE_EUNSUPPORTED;
}

template <int IN>
int launch_mid(int P, const MidParams& p, dim3 grid, int threads, hipStream_t st) {
  switch (P) {
    case 2: return launch_mid_p<2, IN>(p, grid, threads, st);
    case 4: return launch_mid_p<4, IN>(p, grid, threads, st);
    case 6: return launch_mid_p<6, IN>(p, grid, threads, st);
    case 8: return launch_mid_p<8, IN>(p, grid, threads, st);
    case 12: return launch_mid_p<12, IN>(p, grid, threads, st);
    case 16: return launch_mid_p<16, IN>(p, grid, threads, st);
    default: return SPECTRE_EUNSUPPORTED;
  }
}

template <int R, int DT>
int launch_final_r(const FinalParams& p, bool fuse, bool pre, int64_t B, hipStream_t st) {
  if constexpr (R == 48 || R == 64) {
    if (fuse && p.CP2 % 32 == 0) {  // CP2 <= 256 holds whenever fuse does
      const dim3 grid((unsigned)(B * p.M)), block((unsigned)(2 * p.CP2));
      if (p.yblk != nullptr)  // chunked mix (post-norm only)
        hipLaunchKernelGGL((k_final_split<R, DT, false, 1>), grid, block, 0, st, p);
      else if (p.yloc != nullptr && pre)  // local branch
        hipLaunchKernelGGL((k_final_split<R, DT, true, 2>), grid, block, 0, st, p);
      else if (p.yloc != nullptr)
        hipLaunchKernelGGL((k_final_split<R, DT, false, 2>), grid, block, 0, st, p);
      else if (pre)
        hipLaunchKernelGGL((k_final_split<R, DT, true>), grid, block, 0, st, p);
      else
        hipLaunchKernelGGL((k_final_split<R, DT, false>), grid, block, 0, st, p);
      SPECTRE_LAUNCH_CHECK("C1_inv_norm");
      return SPECTRE_OK;
    }
  }
  if (fuse) {
    dim3 grid((unsigned)(B * p.M));
    if (pre)
      hipLaunchKernelGGL((k_final<R, DT, true, true>), grid, dim3((unsigned)p.CP2), 0, st, p);
    else
      hipLaunchKernelGGL((k_final<R, DT, true, false>), grid, dim3((unsigned)p.CP2), 0, st, p);
  } else {
    dim3 grid((unsigned)((p.lines + 255) / 256));
    hipLaunchKernelGGL((k_final<R, DT, false>), grid, dim3(256), 0, st, p);
  }
  SPECTRE_LAUNCH_CHECK(fuse ? "C1_inv_norm" : "C1_inv");
  return SPECTRE_OK;
}

template <int DT>
int launch_final(int64_t R, const FinalParams& p, bool fuse, bool pre, int64_t B, hipStream_t st) {
  switch (R) {
    case 2: return launch_final_r<2, DT>(p, fuse, pre, B, st);
    case 4: return launch_final_r<4, DT>(p, fuse, pre, B, st);
    case 6: return launch_final_r<6, DT>(p, fuse, pre, B, st);
    case 8: return launch_final_r<8, DT>(p, fuse, pre, B, st);
    case 12: return launch_final_r<12, DT>(p, fuse, pre, B, st);
    case 16: return launch_final_r<16, DT>(p, fuse, pre, B, st);
    case 24: return launch_final_r<24, DT>(p, fuse, pre, B, st);
    case 32: return launch_final_r<32, DT>(p, fuse, pre, B, st);
    case 48: return launch_final_r<48, DT>(p, fuse, pre, B, st);
    case 64: return launch_final_r<64, DT>(p, fuse, pre, B, st);
    default: return SPECTRE_EUNSUPPORTED;
  }
}

template <int DT, bool PRE>
int launch_norm_its(const NormParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((p.ntok + 3) / 4)), block(256);
  if (p.CP2 % 2 == 0) {  // two pairs per lane
    if (p.CP2 <= 128) hipLaunchKernelGGL((k_layernorm2<DT, PRE, 1>), grid, block, 0, st, p);
    else if (p.CP2 <= 256) hipLaunchKernelGGL((k_layernorm2<DT, PRE, 2>), grid, block, 0, st, p);
    else if (p.CP2 <= 512) hipLaunchKernelGGL((k_layernorm2<DT, PRE, 4>), grid, block, 0, st, p);
    else if (p.CP2 <= 1024) hipLaunchKernelGGL((k_layernorm2<DT, PRE, 8>), grid, block, 0, st, p);
    else if (p.CP2 <= 2048) hipLaunchKernelGGL((k_layernorm2<DT, PRE, 16>), grid, block, 0, st, p);
    else return SPECTRE_EUNSUPPORTED;
    SPECTRE_LAUNCH_CHECK("LN_norm");
    return SPECTRE_OK;
  }
  if (p.CP2 <= 64) hipLaunchKernelGGL((k_layernorm<DT, PRE, 1>), grid, block, 0, st, p);
  else if (p.CP2 <= 128) hipLaunchKernelGGL((k_layernorm<DT, PRE, 2>), grid, block, 0, st, p);
  else if (p.CP2 <= 256) hipLaunchKernelGGL((k_layernorm<DT, PRE, 4>), grid, block, 0, st, p);
  else if (p.CP2 <= 512) hipLaunchKernelGGL((k_layernorm<DT, PRE, 8>), grid, block, 0, st, p);
  else if (p.CP2 <= 1024) hipLaunchKernelGGL((k_layernorm<DT, PRE, 16>), grid, block, 0, st, p);
  else if (p.CP2 <= 2048) hipLaunchKernelGGL((k_layernorm<DT, PRE, 32>), grid, block, 0, st, p);
  else return SPECTRE_EUNSUPPORTED;
  SPECTRE_LAUNCH_CHECK("LN_norm");
  return SPECTRE_OK;
}

int launch_norm(const NormParams& p, int dtype, bool pre, hipStream_t st) {
  if (dtype == SPECTRE_F32)
    return pre ? launch_norm_its<IN_F32, true>(p, st) : launch_norm_its<IN_F32, false>(p, st);
  return pre ? launch_norm_its<IN_BF16, true>(p, st) : launch_norm_its<IN_BF16, false>(p, st);
}

// The windowed-attention branch over q, k, v of shape s into y (binary32
// [B][L][H][D]).
template <int DT>
int launch_block_d(const LocalParams& p, int64_t D, hipStream_t st) {
  const dim3 grid((unsigned)((p.L + 127) / 128 * p.H * p.B));
  switch (D) {
    case 16: hipLaunchKernelGGL((k_local_attn<DT, 16>), grid, dim3(256), 0, st, p); break;
    case 32: hipLaunchKernelGGL((k_local_attn<DT, 32>), grid, dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL((k_local_attn<DT, 64>), grid, dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((k_local_attn_wide<DT>), grid, dim3(256), 0, st, p); break;
    default: return SPECTRE_EUNSUPPORTED;
  }
  SPECTRE_LAUNCH_CHECK("L_local");
  return SPECTRE_OK;
}

// Head sizes the kernels are built for; item counts and offsets that fit
// their 32-bit arithmetic.
bool local_shape_ok(const Shape& s) {
  if (s.D != 16 && s.D != 32 && s.D != 64 && s.D != 128) return false;
  if (s.L > (int64_t(1) << 30)) return false;
  const int64_t nitem = (s.L + 31) / 32 * s.H * s.B;
  return nitem <= (int64_t)(INT32_MAX / 1024);
}

int launch_local(const void* q, const void* k, const void* v, float* y, const Shape& s,
                 const Local& lw, hipStream_t st) {
  if (!local_shape_ok(s)) return SPECTRE_EUNSUPPORTED;
  LocalParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.y = y;
  p.L = s.L;
  p.B = (int)s.B;
  p.H = (int)s.H;
  p.C = (int)s.C;
  p.WL = (int)std::min<int64_t>(lw.wl, s.L - 1);
  p.WR = (int)std::min<int64_t>(lw.wr, s.L - 1);
  p.scale2 = (float)(1.4426950408889634 / std::sqrt((double)s.D));
  return s.dtype == SPECTRE_F32 ? launch_block_d<IN_F32>(p, s.D, st)
                                : launch_block_d<IN_BF16>(p, s.D, st);
}

// Bytes of the local branch's output (binary32 y_loc) in the workspace.
size_t local_bytes(const Shape& s, const Local* local) {
  return local ? 256 + (size_t)s.N * 4 : 0;
}

// The single-pass column kernel of a ColKind: grid (pair blocks, batch).
template <int RA, int RB, int RC, int CPT, int IN>
int launch_col_k(const ColParams& c, int64_t B, hipStream_t st) {
  using C = ColCfg<RA, RB, RC, CPT>;
  static uint64_t attr_set = 0;  // guarded by g_mu
  if (int rc = lds_attr(reinterpret_cast<const void*>(&k_col<RA, RB, RC, CPT, IN>), (int)C::LDS_BYTES,
                        attr_set))
    return rc;
  const int64_t items = (c.CP2 + CPT - 1) / CPT * B;
  if (items > INT32_MAX) return SPECTRE_EUNSUPPORTED;
  const dim3 grid((unsigned)items);
  hipLaunchKernelGGL((k_col<RA, RB, RC, CPT, IN>), grid, dim3(C::THREADS), C::LDS_BYTES, st, c);
  SPECTRE_LAUNCH_CHECK("B_col");
  return SPECTRE_OK;
}

template <int IN>
int launch_col(int kind, const ColParams& c, int64_t B, hipStream_t st) {
  switch (kind) {
    case COL_3072: return launch_col_k<12, 16, 16, 4, IN>(c, B, st);
    case COL_4096: return launch_col_k<16, 16, 16, 4, IN>(c, B, st);
    default: return SPECTRE_EUNSUPPORTED;
  }
}

// B, the LDS pass, for shape s / plan pl: the column transforms, the
// spectral product and the inverse.  in[] are the raw tensors (single level,
// in_kind their storage) or the spectra (IN_C32); out gets y (single level)
// or U; gtab is the gate table of a multi-level square kernel, else null;
// dc (chunked mix) receives the block means; resid (column kernel only) is
// added to y before it is stored.
int launch_b(const Shape& s, const Plan& pl, const LenTables* tab, const void* const in[3],
             int in_kind, float2* out, const float* gate, const float* gtab, int tiled,
             float2* dc, hipStream_t st, const void* resid = nullptr) {
  const bool single = is_single(pl);
  const int64_t CP2 = s.CP2;
  MidParams m{};
  const int nslot = single ? 1 : 2;
  const int cpt = pl.sq ? choose_cpt_sq(pl.sq, CP2, nslot) : choose_cpt(pl, CP2, nslot);
  for (int t = 0; t < 3; ++t) m.in[t] = in[t];
  m.out = out;
  m.tiled = tiled;
  m.gate = gate;
  m.gate_kind = s.gate_kind;
  m.gtab = gtab;
  m.ncol = (int)(pl.L1 * pl.L2);
  m.twN = tab->twN;
  m.twL = tab->twL;
  m.wgcols = tab->wgcols;
  m.L = (int)s.L;
  m.L1 = (int)pl.L1;
  m.L2 = (int)pl.L2;
  m.N = (int)pl.L3;
  m.M = (int)(pl.L2 * pl.L3);
  m.CP2 = (int)CP2;
  m.D = (int)s.D;
  m.keep = (int)s.keep;
  m.nbins = (int)(s.L / 2 + 1);
  m.nslot = nslot;
  m.cpt = cpt;
  m.Tc = pl.Tc;
  m.selfwg = tab->selfwg;
  m.nrad = pl.nrad;
  for (int i = 0; i < 8; ++i) m.rad[i] = pl.rad[i];
  m.scale = (float)(1.0 / (8.0 * (double)s.L * (double)s.L));
  m.dc = dc;
  m.dc_stride = s.B * CP2;
  m.dc_scale = (float)(1.0 / (double)s.L);
  if (pl.col) {
    ColParams c{};
    for (int t = 0; t < 3; ++t) c.in[t] = in[t];
    c.x = resid;
    c.out = out;
    c.gate = gate;
    c.tw = tab->twN;
    c.gate_kind = s.gate_kind;
    c.CP2 = (int)CP2;
    c.D = (int)s.D;
    c.keep = (int)s.keep;
    c.nbins = (int)(s.L / 2 + 1);
    c.scale = m.scale;
    c.dc = dc;
    c.dc_stride = m.dc_stride;
    c.dc_scale = m.dc_scale;
    return in_kind == IN_BF16 ? launch_col<IN_BF16>(pl.col, c, s.B, st)
                              : launch_col<IN_F32>(pl.col, c, s.B, st);
  }
  dim3 grid((unsigned)tab->nwg, (unsigned)(CP2 / cpt), (unsigned)s.B);
  const int threads = pl.Tc * nslot * cpt;
  if (pl.sq) {
    if (in_kind == IN_F32) return launch_mid_square<IN_F32>(pl.sq, m, grid, st);
    if (in_kind == IN_BF16) return launch_mid_square<IN_BF16>(pl.sq, m, grid, st);
    return launch_mid_square<IN_C32>(pl.sq, m, grid, st);
  }
  if (in_kind == IN_F32) return launch_mid<IN_F32>(pl.P, m, grid, threads, st);
  if (in_kind == IN_BF16) return launch_mid<IN_BF16>(pl.P, m, grid, threads, st);
  return launch_mid<IN_C32>(pl.P, m, grid, threads, st);
}

// The chunked mix's inter-block step: the block means dc ([3][B][nb][pairs],
// binary32) mixed over the block axis -- a single-level mix of length nb
// with gate_blocks -- into yblk ([B][nb][pairs]).
int launch_block_mix(int dev, const Shape& s, const Chunk& ch, const float2* dc, float2* yblk,
                     hipStream_t st) {
  Shape sb = s;
  sb.B = ch.B;
  sb.L = ch.nb;
  sb.N = ch.B * ch.nb * s.C;
  sb.keep = ch.keep_blocks;
  sb.dtype = SPECTRE_F32;
  sb.esz = 4;
  sb.gate_kind = SPECTRE_GATE_REAL;
  Plan pb;
  int rc = make_plan(ch.nb, pb, col_fits(ch.B, s.CP2));
  if (rc) return rc;
  if (!is_single(pb)) return SPECTRE_EUNSUPPORTED;
  LenTables* tb = nullptr;
  rc = get_tables(dev, pb, &tb);
  if (rc) return rc;
  const int64_t per = ch.B * ch.nb * s.CP2;  // pairs per tensor of block means
  const void* ins[3] = {dc, dc + per, dc + 2 * per};
  return launch_b(sb, pb, tb, ins, IN_F32, yblk, ch.gate_blocks, nullptr, 0, nullptr, st);
}

// The spectral part into `y` (pairs, binary32), and optionally the fused
// residual + LayerNorm into `out`.
int launch_all(int dev, const void* q, const void* k, const void* v, const void* x,
               const float* gate, const float* gamma, const float* beta, void* out, float* y,
               const Shape& s, const Plan& pl, const LenTables* tab, void* ws, hipStream_t st,
               const Chunk* chunk, const Local* local);

int run(const void* q, const void* k, const void* v, const void* x, const float* gate,
        const float* gamma, const float* beta, void* out, float* y, const Shape& s,
        const Plan& pl, hipStream_t st, const Chunk* chunk = nullptr,
        const Local* local = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPECTRE_EHIP;
  std::lock_guard<std::mutex> lock(g_mu);
  LenTables* tab = nullptr;
  int rc = get_tables(dev, pl, &tab);
  if (rc) return rc;
  const bool want_out = out != nullptr;
  void* ws = nullptr;
  const size_t wsb = workspace_for(s, pl, want_out) + chunk_bytes(s, chunk) + local_bytes(s, local);
  if (wsb) {
    rc = get_workspace(dev, wsb, &ws);
    if (rc) return rc;
  }
  return launch_all(dev, q, k, v, x, gate, gamma, beta, out, y, s, pl, tab, ws, st, chunk, local);
}

// Every launch of one call, given its tables and workspace (g_mu held).
int launch_all(int dev, const void* q, const void* k, const void* v, const void* x,
               const float* gate, const float* gamma, const float* beta, void* out, float* y,
               const Shape& s, const Plan& pl, const LenTables* tab, void* ws, hipStream_t st,
               const Chunk* chunk, const Local* local) {
  int rc = SPECTRE_OK;
  const bool want_out = out != nullptr;
  // local branch: y_loc after the rest, computed first and added by the norm
  float2* yloc = local ? reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) +
                                                   ((workspace_for(s, pl, want_out) + 255) & ~(size_t)255))
                       : nullptr;
  // chunked mix: the block means of q, k, v and the block term, after the rest
  float2* dc = chunk ? reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) +
                                                 ((workspace_for(s, pl, want_out) + 255) & ~(size_t)255))
                     : nullptr;
  float2* yblk = chunk ? dc + 3 * s.B * s.CP2 : nullptr;
  trace_call_begin(st);
  if (local) {
    rc = launch_local(q, k, v, reinterpret_cast<float*>(yloc), s, *local, st);
    if (rc) return rc;
  }
  const int64_t CP2 = s.CP2;
  const int64_t pairs = s.B * s.L * CP2;  // complex elements per tensor
  const int in_kind = s.dtype == SPECTRE_F32 ? IN_F32 : IN_BF16;
  const bool single = is_single(pl);
  float2* T = reinterpret_cast<float2*>(ws);  // [3][B][L][CP2] complex (multi-level)
  const bool tiled = tiled_plan(s, pl);
  const bool tiled3 = tiled3_plan(s, pl);
  float2* U = tiled ? T + 3 * pairs : T;       // B's output, row layout
  float2* S = tiled3 ? T + 3 * pairs : T;      // the spectra B reads

  // ---- gate table of the square B kernel: scale, truncation and the mirror
  // bin folded in, laid out [h][column][k3] so B's lanes read it coalesced;
  // built by an extra grid plane of the first pass for multi-level plans
  GateTabParams g{};
  if (pl.sq && !single) {
    g.gate = gate;
    g.gtab = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                      ((spectra_bytes(s, pl, want_out) + 255) & ~(size_t)255));
    g.L = s.L;
    g.L1 = (int)pl.L1;
    g.L2 = (int)pl.L2;
    g.N = (int)pl.L3;
    g.ncol = (int)(pl.L1 * pl.L2);
    g.nbins = (int)(s.L / 2 + 1);
    g.keep = s.keep;
    g.total = s.H * s.L;
    g.scale = (float)(1.0 / (8.0 * (double)s.L * (double)s.L));
    g.kind = s.gate_kind;
  }
  const bool gate_in_a1 = g.gtab != nullptr;  // multi-level square B: A1 builds the table

  // ---- forward strided passes
  if (!single) {
    StridedParams a1{};
    if (gate_in_a1) a1.gt = g;
    a1.in[0] = q;
    a1.in[1] = k;
    a1.in[2] = v;
    for (int t = 0; t < 3; ++t) a1.out[t] = T + t * pairs;
    a1.twL = tab->twL;
    a1.outer = s.B;
    a1.inner = pl.L2 * pl.L3;
    a1.CP2 = CP2;
    a1.L1 = (int)pl.L1;
    rc = in_kind == IN_F32 ? strided_fwd<IN_F32>(pl.L1, a1, TW_A1, 3, st, tiled)
                           : strided_fwd<IN_BF16>(pl.L1, a1, TW_A1, 3, st, tiled);
    if (rc) return rc;
    if (pl.L2 > 1) {
      StridedParams a2{};
      for (int t = 0; t < 3; ++t) {
        a2.in[t] = T + t * pairs;
        a2.out[t] = S + t * pairs;
      }
      a2.twL = tab->twL;
      a2.outer = s.B * pl.L1;
      a2.inner = pl.L3;
      a2.CP2 = CP2;
      a2.L1 = (int)pl.L1;
      rc = strided_fwd<IN_C32>(pl.L2, a2, TW_A2, 3, st, tiled3);
      if (rc) return rc;
    }
  }

  // ---- B: LDS transform, spectral product, inverse.  The column kernel of a
  // post-norm call without the local branch stores x + y, so that the norm
  // pass reads one tensor instead of two
  const bool fold_x = pl.col && want_out && (s.norm_order & 1) == 0 && !local;
  {
    const void* ins[3] = {q, k, v};
    if (!single)
      for (int t = 0; t < 3; ++t) ins[t] = S + t * pairs;
    float2* bout = single ? (want_out ? reinterpret_cast<float2*>(ws) : reinterpret_cast<float2*>(y))
                          : U;  // row layout: q's spectrum in place, unless tiled
    rc = launch_b(s, pl, tab, ins, single ? in_kind : IN_C32, bout, gate, g.gtab,
                  tiled || tiled3 ? 1 : 0, chunk ? dc : nullptr, st, fold_x ? x : nullptr);
    if (rc) return rc;
  }

  // ---- chunked mix: the block means, mixed over the block axis, into yblk
  if (chunk) {
    rc = launch_block_mix(dev, s, *chunk, dc, yblk, st);
    if (rc) return rc;
    trace_rename_last("B_block_axis");
    if (single && !want_out) {  // y only, written by B: add the block term here
      const int64_t n = s.B * s.L * CP2;
      const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
      hipLaunchKernelGGL(k_block_add, dim3((unsigned)blocks), dim3(256), 0, st,
                         reinterpret_cast<float2*>(y), yblk, n, s.L, CP2);
      SPECTRE_LAUNCH_CHECK("block_add");
      return SPECTRE_OK;
    }
  }

  const float inv_c = (float)(1.0 / (double)s.C);
  const float eps = 1e-5f;
  const bool pre = (s.norm_order & 1) != 0;  // bit 0: order, bit 1: RMSNorm
  const int rms = (s.norm_order & 2) != 0 ? 1 : 0;
  const float* mix = local ? local->mix : nullptr;
  if (single) {
    if (!want_out) return SPECTRE_OK;
    NormParams n{};
    n.y = reinterpret_cast<const float2*>(ws);
    n.x = fold_x ? nullptr : x;
    n.gamma = gamma;
    n.beta = beta;
    n.out = out;
    n.ntok = s.B * s.L;
    n.CP2 = CP2;
    n.inv_c = inv_c;
    n.eps = eps;
    n.yblk = yblk;  // chunked mix: the block term joins y here
    n.Lb = s.L;
    n.yloc = yloc;  // local branch: joins y here
    n.mix = mix;
    n.rms = rms;
    return launch_norm(n, s.dtype, pre, st);
  }

  // ---- inverse strided passes
  if (pl.L2 > 1) {
    StridedParams c2{};
    c2.in[0] = T;
    c2.out[0] = T;
    c2.twL = tab->twL;
    c2.outer = s.B * pl.L1;
    c2.inner = pl.L3;
    c2.CP2 = CP2;
    c2.L1 = (int)pl.L1;
    rc = strided_inv(pl.L2, c2, st);
    if (rc) return rc;
  }
  const bool fuse = want_out && fused_norm_ok(CP2);
  FinalParams f{};
  f.U = U;
  f.x = x;
  f.gamma = gamma;
  f.beta = beta;
  f.M = pl.L2 * pl.L3;
  f.CP2 = CP2;
  f.L = s.L;
  f.lines = s.B * f.M * CP2;
  f.inv_c = inv_c;
  f.eps = eps;
  f.yblk = yblk;  // chunked mix: the block term joins y in C1
  f.yloc = fuse ? yloc : nullptr;  // local branch: joins y in the fused C1, else in the norm
  f.mix = mix;
  f.rms = rms;
  // y for a separate LayerNorm: k's spectrum region is free once B has run
  float* ybuf = want_out ? reinterpret_cast<float*>(T + pairs) : y;
  if (fuse) {
    f.out = out;
    return s.dtype == SPECTRE_F32 ? launch_final<IN_F32>(pl.L1, f, true, pre, s.B, st)
                                  : launch_final<IN_BF16>(pl.L1, f, true, pre, s.B, st);
  }
  f.out = ybuf;
  rc = launch_final<IN_F32>(pl.L1, f, false, false, s.B, st);
  if (rc || !want_out) return rc;

  NormParams n{};
  n.y = reinterpret_cast<const float2*>(ybuf);
  n.x = x;
  n.gamma = gamma;
  n.beta = beta;
  n.out = out;
  n.ntok = s.B * s.L;
  n.CP2 = CP2;
  n.inv_c = inv_c;
  n.eps = eps;
  n.yloc = yloc;
  n.mix = mix;
  n.rms = rms;
  return launch_norm(n, s.dtype, pre, st);
}

// Validates a chunked call: the blockwise shape (B * nb batches of fft_len
// tokens) and the block axis (nb = L / fft_len, even, one-level plan).
int check_chunked(int64_t B, int64_t H, int64_t L, int64_t D, int64_t fft_len, int64_t keep_bins,
                  int64_t keep_blocks, int dtype, Shape& s, Plan& pl, Chunk& ch) {
  if (B < 1 || L < 2 || fft_len < 2) return SPECTRE_EINVAL;
  if (L % fft_len != 0) return SPECTRE_EINVAL;
  const int64_t nb = L / fft_len;
  if (nb % 2 != 0 || keep_blocks < 0 || keep_blocks > nb / 2 + 1) return SPECTRE_EINVAL;
  if (B > (int64_t(1) << 40) / L) return SPECTRE_EUNSUPPORTED;
  int rc = check_shape(B * nb, H, fft_len, D, keep_bins, dtype, s, pl);
  if (rc) return rc;
  Plan pb;
  rc = make_plan(nb, pb, col_fits(B, s.CP2));  // as launch_block_mix plans it
  if (rc) return rc;
  if (!is_single(pb)) return SPECTRE_EUNSUPPORTED;
  ch.nb = nb;
  ch.keep_blocks = keep_blocks;
  ch.B = B;
  return SPECTRE_OK;
}

// The mix with the local branch, summed (mix null) or gated per channel.
int local_call(const void* q, const void* k, const void* v, const void* x, const float* gate,
               const float* mix, const float* gamma, const float* beta, void* out, int64_t B,
               int64_t H, int64_t L, int64_t D, int64_t keep_bins, int64_t win_left,
               int64_t win_right, int dtype, int gate_kind, int norm_order, hipStream_t stream) {
  if (!q || !k || !v || !x || !gate || !gamma || !beta || !out) return SPECTRE_EINVAL;
  if (win_left < 0 || win_right < 0) return SPECTRE_EINVAL;
  Shape s;
  Plan pl;
  int rc = check_shape(B, H, L, D, keep_bins, dtype, s, pl, gate_kind, norm_order);
  if (rc) return rc;
  if (!local_shape_ok(s)) return SPECTRE_EUNSUPPORTED;
  const void* ptrs[] = {q, k, v, x, gate, gamma, beta, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECTRE_EINVAL;
  const size_t tb = (size_t)s.N * s.esz;
  for (const void* p : {q, k, v, x})
    if (overlaps(out, tb, p, tb)) return SPECTRE_EINVAL;
  const Local lw{win_left, win_right, mix};
  return run(q, k, v, x, gate, gamma, beta, out, nullptr, s, pl, stream, nullptr, &lw);
}

// ------------------------------------------- allocation-free entry point
//
// spectre_mix_fwd_noalloc keeps its workspace and tables in `scratch`, a
// file-scope device array of kNoAllocBytes that every GPU the library runs
// on holds until the process ends.  In host code the array's name is only a
// stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress (once per device, with that device current) and is the
// only handle used for it.  Every call on one GPU shares that GPU's array, so
// calls that overlap on one GPU race.  Layout: the workspace of
// spectre_mix_fwd (spectra, gate table), then the twiddles w_L^e, e < L, the
// twiddles w_N^e, e < N, and B's column pairs, each 256-byte aligned and all
// written by every call before they are read (nothing needs clearing).

constexpr size_t kNoAllocBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocBytes];
void* g_scratch[kMaxDevices] = {nullptr};  // per device; guarded by g_mu

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The tables of a one- or two-level plan: w_L^e (e < L), w_N^e (e < N) and
// B's column pairs -- (0, -1) for one level; for two levels (L2 = 1) the
// pairs (k1, L1 - k1), k1 = 1 .. L1/2 - 1, then the self-paired columns
// (0, L1/2), the order build_wgcols gives.
__global__ void k_build_tables(float2* twL, int64_t L, float2* twN, int64_t N, int2* wgcols,
                               int nwg, int L1, int single) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < L) twL[i] = host_twiddle(i, L);
  if (i < N) twN[i] = host_twiddle(i, N);
  if (i < nwg) {
    const int c = (int)i;
    wgcols[i] = single ? make_int2(0, -1) : c < L1 / 2 - 1 ? make_int2(c + 1, L1 - 1 - c) : make_int2(0, L1 / 2);
  }
}

}  // namespace
}  // namespace spectre

using namespace spectre;

extern "C" {

int spectre_mix_fwd_ex(const void* q, const void* k, const void* v, const void* x,
                       const float* gate, const float* gamma, const float* beta, void* out,
                       int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins, int dtype,
                       int gate_kind, int norm_order, hipStream_t stream) {
  if (!q || !k || !v || !x || !gate || !gamma || !beta || !out) return SPECTRE_EINVAL;
  Shape s;
  Plan pl;
  int rc = check_shape(B, H, L, D, keep_bins, dtype, s, pl, gate_kind, norm_order);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, x, gate, gamma, beta, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECTRE_EINVAL;
  const size_t tb = (size_t)s.N * s.esz;
  for (const void* p : {q, k, v, x})
    if (overlaps(out, tb, p, tb)) return SPECTRE_EINVAL;
  return run(q, k, v, x, gate, gamma, beta, out, nullptr, s, pl, stream);
}

int spectre_mix_fwd(const void* q, const void* k, const void* v, const void* x, const float* gate,
                    const float* gamma, const float* beta, void* out, int64_t B, int64_t H,
                    int64_t L, int64_t D, int64_t keep_bins, int dtype, hipStream_t stream) {
  return spectre_mix_fwd_ex(q, k, v, x, gate, gamma, beta, out, B, H, L, D, keep_bins, dtype,
                            SPECTRE_GATE_REAL, SPECTRE_NORM_POST, stream);
}

int spectre_mix_fwd_noalloc(const void* q, const void* k, const void* v, const void* x,
                            const float* gate, const float* gamma, const float* beta, void* out,
                            int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins,
                            int dtype, hipStream_t stream) {
  if (!q || !k || !v || !x || !gate || !gamma || !beta || !out) return SPECTRE_EINVAL;
  Shape s;
  Plan pl;
  int rc = check_shape(B, H, L, D, keep_bins, dtype, s, pl);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, x, gate, gamma, beta, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECTRE_EINVAL;
  const size_t tb = (size_t)s.N * s.esz;
  for (const void* p : {q, k, v, x})
    if (overlaps(out, tb, p, tb)) return SPECTRE_EINVAL;
  // one- and two-level plans only; everything must fit the scratch array
  const bool single = is_single(pl);
  if (!single && pl.L2 != 1) return SPECTRE_EUNSUPPORTED;
  const int nwg = single ? 1 : (int)(pl.L1 / 2);
  const size_t o_twl = align256(workspace_for(s, pl, true));
  const size_t o_twn = o_twl + align256(sizeof(float2) * (size_t)pl.L);
  const size_t o_wg = o_twn + align256(sizeof(float2) * (size_t)pl.L3);
  if (o_wg + align256(sizeof(int2) * (size_t)nwg) > kNoAllocBytes) return SPECTRE_EUNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPECTRE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SPECTRE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {  // set-up, once per device: this GPU's copy of the array
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return SPECTRE_EHIP;
    g_scratch[dev] = ptr;
  }
  char* base = static_cast<char*>(g_scratch[dev]);
  LenTables t;
  t.twL = reinterpret_cast<float2*>(base + o_twl);
  t.twN = reinterpret_cast<float2*>(base + o_twn);
  t.wgcols = reinterpret_cast<int2*>(base + o_wg);
  t.nwg = nwg;
  t.selfwg = single ? -1 : nwg - 1;
  const int64_t n = std::max<int64_t>(pl.L, nwg);
  hipLaunchKernelGGL(k_build_tables, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, t.twL,
                     (int64_t)pl.L, t.twN, (int64_t)pl.L3, t.wgcols, nwg, (int)pl.L1, single ? 1 : 0);
  if (hipGetLastError() != hipSuccess) return SPECTRE_EHIP;
  return launch_all(dev, q, k, v, x, gate, gamma, beta, out, nullptr, s, pl, &t, base, stream, nullptr,
                    nullptr);
}

int spectre_mix_y_ex(const void* q, const void* k, const void* v, const float* gate, float* y,
                     int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins, int dtype,
                     int gate_kind, hipStream_t stream) {
  if (!q || !k || !v || !gate || !y) return SPECTRE_EINVAL;
  Shape s;
  Plan pl;
  int rc = check_shape(B, H, L, D, keep_bins, dtype, s, pl, gate_kind, SPECTRE_NORM_POST);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, gate, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECTRE_EINVAL;
  const size_t tb = (size_t)s.N * s.esz;
  for (const void* p : {q, k, v})
    if (overlaps(y, (size_t)s.N * 4, p, tb)) return SPECTRE_EINVAL;
  return run(q, k, v, nullptr, gate, nullptr, nullptr, nullptr, y, s, pl, stream);
}

int spectre_mix_y(const void* q, const void* k, const void* v, const float* gate, float* y,
                  int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins, int dtype,
                  hipStream_t stream) {
  return spectre_mix_y_ex(q, k, v, gate, y, B, H, L, D, keep_bins, dtype, SPECTRE_GATE_REAL,
                          stream);
}

int spectre_mix_fwd_chunked(const void* q, const void* k, const void* v, const void* x,
                            const float* gate, const float* gate_blocks, const float* gamma,
                            const float* beta, void* out, int64_t B, int64_t H, int64_t L, int64_t D,
                            int64_t fft_len, int64_t keep_bins, int64_t keep_blocks, int dtype,
                            hipStream_t stream) {
  if (!q || !k || !v || !x || !gate || !gate_blocks || !gamma || !beta || !out)
    return SPECTRE_EINVAL;
  Shape s;
  Plan pl;
  Chunk ch{};
  int rc = check_chunked(B, H, L, D, fft_len, keep_bins, keep_blocks, dtype, s, pl, ch);
  if (rc) return rc;
  ch.gate_blocks = gate_blocks;
  const void* ptrs[] = {q, k, v, x, gate, gate_blocks, gamma, beta, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECTRE_EINVAL;
  const size_t tb = (size_t)s.N * s.esz;
  for (const void* p : {q, k, v, x})
    if (overlaps(out, tb, p, tb)) return SPECTRE_EINVAL;
  return run(q, k, v, x, gate, gamma, beta, out, nullptr, s, pl, stream, &ch);
}

int spectre_mix_y_chunked(const void* q, const void* k, const void* v, const float* gate,
                          const float* gate_blocks, float* y, int64_t B, int64_t H, int64_t L,
                          int64_t D, int64_t fft_len, int64_t keep_bins, int64_t keep_blocks,
                          int dtype, hipStream_t stream) {
  if (!q || !k || !v || !gate || !gate_blocks || !y) return SPECTRE_EINVAL;
  Shape s;
  Plan pl;
  Chunk ch{};
  int rc = check_chunked(B, H, L, D, fft_len, keep_bins, keep_blocks, dtype, s, pl, ch);
  if (rc) return rc;
  ch.gate_blocks = gate_blocks;
  const void* ptrs[] = {q, k, v, gate, gate_blocks, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECTRE_EINVAL;
  const size_t tb = (size_t)s.N * s.esz;
  for (const void* p : {q, k, v})
    if (overlaps(y, (size_t)s.N * 4, p, tb)) return SPECTRE_EINVAL;
  return run(q, k, v, nullptr, gate, nullptr, nullptr, nullptr, y, s, pl, stream, &ch);
}

int spectre_mix_fwd_local_gated(const void* q, const void* k, const void* v, const void* x,
                                const float* gate, const float* mix, const float* gamma,
                                const float* beta, void* out, int64_t B, int64_t H, int64_t L,
                                int64_t D, int64_t keep_bins, int64_t win_left, int64_t win_right,
                                int dtype, int gate_kind, int norm_order, hipStream_t stream) {
  if (!mix || !aligned16(mix)) return SPECTRE_EINVAL;
  return local_call(q, k, v, x, gate, mix, gamma, beta, out, B, H, L, D, keep_bins, win_left,
                    win_right, dtype, gate_kind, norm_order, stream);
}

int spectre_mix_fwd_local_ex(const void* q, const void* k, const void* v, const void* x,
                             const float* gate, const float* gamma, const float* beta, void* out,
                             int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins,
                             int64_t win_left, int64_t win_right, int dtype, int gate_kind,
                             int norm_order, hipStream_t stream) {
  return local_call(q, k, v, x, gate, nullptr, gamma, beta, out, B, H, L, D, keep_bins, win_left,
                    win_right, dtype, gate_kind, norm_order, stream);
}

int spectre_mix_fwd_local(const void* q, const void* k, const void* v, const void* x,
                          const float* gate, const float* gamma, const float* beta, void* out,
                          int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins,
                          int64_t win_left, int64_t win_right, int dtype, hipStream_t stream) {
  return spectre_mix_fwd_local_ex(q, k, v, x, gate, gamma, beta, out, B, H, L, D, keep_bins,
                                  win_left, win_right, dtype, SPECTRE_GATE_REAL, SPECTRE_NORM_POST,
                                  stream);
}

int spectre_mix_local_attention(const void* q, const void* k, const void* v, float* y, int64_t B,
                                int64_t H, int64_t L, int64_t D, int64_t win_left,
                                int64_t win_right, int dtype, hipStream_t stream) {
  if (!q || !k || !v || !y) return SPECTRE_EINVAL;
  if (win_left < 0 || win_right < 0) return SPECTRE_EINVAL;
  if (B < 1 || H < 1 || D < 1 || L < 1) return SPECTRE_EINVAL;
  if (dtype != SPECTRE_F32 && dtype != SPECTRE_BF16) return SPECTRE_EINVAL;
  if (H > kMaxC || D > kMaxC || H * D > kMaxC) return SPECTRE_EUNSUPPORTED;
  if (L > (int64_t(1) << 40) / (B * H * D)) return SPECTRE_EUNSUPPORTED;
  Shape s{};
  s.B = B;
  s.H = H;
  s.L = L;
  s.D = D;
  s.C = H * D;
  s.N = B * L * H * D;
  s.dtype = dtype;
  s.esz = dtype == SPECTRE_F32 ? 4 : 2;
  if (!local_shape_ok(s)) return SPECTRE_EUNSUPPORTED;
  const void* ptrs[] = {q, k, v, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECTRE_EINVAL;
  const size_t tb = (size_t)s.N * s.esz;
  for (const void* p : {q, k, v})
    if (overlaps(y, (size_t)s.N * 4, p, tb)) return SPECTRE_EINVAL;
  std::lock_guard<std::mutex> lock(g_mu);
  trace_call_begin(stream);
  return launch_local(q, k, v, y, s, Local{win_left, win_right}, stream);
}

size_t spectre_mix_workspace_bytes_ex(int64_t B, int64_t H, int64_t L, int64_t D, int dtype,
                                      int gate_kind) {
  Shape s;
  Plan pl;
  if (check_shape(B, H, L, D, 0, dtype, s, pl, gate_kind, SPECTRE_NORM_POST) != SPECTRE_OK)
    return 0;
  return workspace_for(s, pl, true);
}

size_t spectre_mix_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D, int dtype) {
  return spectre_mix_workspace_bytes_ex(B, H, L, D, dtype, SPECTRE_GATE_REAL);
}

int spectre_mix_plan(int64_t L, int64_t* l1, int64_t* l2, int64_t* l3) {
  if (!l1 || !l2 || !l3) return SPECTRE_EINVAL;
  Plan pl;
  int rc = make_plan(L, pl);
  if (rc) return rc;
  *l1 = pl.L1;
  *l2 = pl.L2;
  *l3 = pl.L3;
  return SPECTRE_OK;
}

int spectre_mix_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int cur = 0;
  bool have_cur = hipGetDevice(&cur) == hipSuccess;
  int rc = SPECTRE_OK;
  for (auto& kv : g_dev) {
    if (hipSetDevice(kv.first) != hipSuccess) {
      rc = SPECTRE_EHIP;
      continue;
    }
    DeviceState& ds = kv.second;
    if (ds.ws && hipFree(ds.ws) != hipSuccess) rc = SPECTRE_EHIP;
    ds.ws = nullptr;
    ds.ws_bytes = 0;
    for (auto& t : ds.tables) {
      if (hipFree(t.second.twL) != hipSuccess) rc = SPECTRE_EHIP;
      if (hipFree(t.second.twN) != hipSuccess) rc = SPECTRE_EHIP;
      if (hipFree(t.second.wgcols) != hipSuccess) rc = SPECTRE_EHIP;
    }
    ds.tables.clear();
  }
  g_dev.clear();
  if (have_cur) (void)hipSetDevice(cur);
  return rc;
}

int spectre_mix_trace_start(int max_calls) {
  if (max_calls < 1 || max_calls > 100000) return SPECTRE_EINVAL;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_trace.on) return SPECTRE_EINVAL;
  const size_t n = (size_t)max_calls * (kMaxKernelsPerCall + 1);
  g_trace = TraceState();
  g_trace.pool.resize(n);
  for (size_t i = 0; i < n; ++i) {
    if (hipEventCreate(&g_trace.pool[i]) != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(g_trace.pool[j]);
      g_trace = TraceState();
      return SPECTRE_EHIP;
    }
  }
  g_trace.on = true;
  g_trace.max_calls = max_calls;
  return SPECTRE_OK;
}

int spectre_mix_trace_stop(int max_kernels, float* total_ms, int* n_kernels, int* n_calls,
                           char* names, int name_len) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_trace.on) return SPECTRE_EINVAL;
  int rc = SPECTRE_OK;
  const int nk = g_trace.calls.empty() ? 0 : g_trace.calls[0].nk;
  for (const TraceCall& c : g_trace.calls)
    if (c.nk != nk) rc = SPECTRE_EINVAL;
  if (g_trace.used > 0 && hipEventSynchronize(g_trace.pool[g_trace.used - 1]) != hipSuccess)
    rc = SPECTRE_EHIP;
  if (rc == SPECTRE_OK) {
    if (nk > max_kernels || !total_ms || !n_kernels || !n_calls) {
      rc = SPECTRE_EINVAL;
    } else {
      for (int k = 0; k < nk; ++k) total_ms[k] = 0.f;
      for (const TraceCall& c : g_trace.calls)
        for (int k = 0; k < nk; ++k) {
          float ms = 0.f;
          if (hipEventElapsedTime(&ms, g_trace.pool[c.first + k], g_trace.pool[c.first + k + 1]) !=
              hipSuccess)
            rc = SPECTRE_EHIP;
          total_ms[k] += ms;
        }
      *n_kernels = nk;
      *n_calls = (int)g_trace.calls.size();
      if (names && name_len > 0 && !g_trace.calls.empty())
        for (int k = 0; k < nk; ++k) {
          std::strncpy(names + (size_t)k * name_len, g_trace.calls[0].names[k], name_len - 1);
          names[(size_t)k * name_len + name_len - 1] = 0;
        }
    }
  }
  for (hipEvent_t e : g_trace.pool) (void)hipEventDestroy(e);
  g_trace = TraceState();
  return rc;
}

const char* spectre_mix_strerror(int status) {
  switch (status) {
    case SPECTRE_OK: return "success";
    case SPECTRE_EINVAL: return "invalid argument";
    case SPECTRE_EUNSUPPORTED: return "unsupported shape";
    case SPECTRE_ENOMEM: return "out of device memory";
    case SPECTRE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
