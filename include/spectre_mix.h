/*
 * spectre_mix.h -- C ABI of the MI355X (gfx950) SPECTRE spectral-mix library.
 *
 * The operation (SPECTRE FFT-attention article, hotelren.com/news/5925787:
 * section 2.2 and its pseudocode for the transform / cross-spectrum / gate /
 * inverse / residual-norm order; section 2.3 for keeping only the first
 * frequency bins; section 3.1 for treating re/im as two real channels):
 *
 *   for each batch b, head h, channel d (one "column" of length L):
 *     Q[f] = sum_{n<L} q[b,n,h,d] exp(-2 pi i f n / L),  f = 0 .. L/2   (same for K, V)
 *     O[f] = (G[h][f] / L) * Q[f] * conj(K[f]) * V[f]   if f < keep_bins, else 0
 *     y[b,t,h,d] = inverse real FFT of O along the sequence (1/L normalisation,
 *                  imaginary parts of bins 0 and L/2 dropped)
 *   out[b,t,:] = LayerNorm over the H*D channels of (x[b,t,:] + y[b,t,:]):
 *                (z - mean) / sqrt(var + 1e-5) * gamma + beta, biased variance.
 *
 * Everything runs in hand-written HIP kernels on the GPU; the host code only
 * validates arguments, plans the transform, manages the workspace and
 * enqueues kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors q, k, v, x, out: layout [B, L, H, D], contiguous, D fastest,
 *    storage type `dtype` (SPECTRE_F32: IEEE binary32; SPECTRE_BF16: bfloat16,
 *    stored as 16-bit patterns, rounded to nearest-even on output).  All
 *    arithmetic is binary32.
 *  - gate: [H][L/2 + 1] binary32, a real multiplier per (head, bin), shared
 *    over b and d.  Values at bins at or above keep_bins are ignored.
 *  - gamma, beta: [H*D] binary32.
 *  - All tensor pointers are DEVICE pointers on the current HIP device and
 *    must be 16-byte aligned.  The caller owns them; the library never frees
 *    or retains them past the call's stream work.
 *  - Calls are asynchronous and stream-ordered on `stream` (0 = the null
 *    stream): inputs must stay valid until the stream reaches the work.
 *    Execution faults surface at the caller's next synchronisation.
 *  - Argument validation happens before any device call; on any error code
 *    nothing is enqueued and `out` is untouched.
 *  - The library owns a per-device workspace and per-(device, plan) twiddle
 *    tables, created lazily on first use (so the first call on a device
 *    allocates device memory), guarded by a mutex, reused by later calls,
 *    and freed by spectre_mix_release().  Two calls that overlap in time on
 *    different streams of one device share that workspace and race: order
 *    them on one stream, or give each its own process.
 *
 * Supported shapes
 * ----------------
 *  B, H, D >= 1; H*D even and at most 4096; L even, L = 2^a * 3^b with
 *  b <= 1 and 2 <= L <= 3 * 2^20 (other lengths: SPECTRE_EUNSUPPORTED; odd L:
 *  SPECTRE_EINVAL);
 *  0 <= keep_bins <= L/2 + 1 (keep_bins = L/2 + 1: no truncation;
 *  keep_bins = 0: y = 0, out = LayerNorm(x)).  L*H*D must be below 2^29 (one
 *  batch element's q spectrum under 4 GiB) and B*L*H*D below 2^40.
 */
#ifndef SPECTRE_MIX_H
#define SPECTRE_MIX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SPECTRE_F32 = 0, SPECTRE_BF16 = 1 } spectre_dtype;

/*
 * How the gate array is read (the *_ex entry points; the others use REAL).
 *  SPECTRE_GATE_REAL:    gate [H][L/2+1] f32, the real multiplier G[h][f]
 *                        (the article's section 2.2, a learnable G(f)).
 *  SPECTRE_GATE_LOGIT:   gate [H][L/2+1] f32 holds logits a; the multiplier is
 *                        the logistic sigmoid 1 / (1 + exp(-a)), computed in
 *                        binary32 (section 3.1 recommends a sigmoid gate).
 *  SPECTRE_GATE_COMPLEX: gate [H][L/2+1][2] f32, the real and imaginary parts
 *                        of a complex multiplier (section 2.4 carries relative
 *                        position as a frequency-dependent rotation factor in
 *                        G(f)).  Bins above L/2 use its conjugate (the output
 *                        stays real), and at bins 0 and L/2 only its real part
 *                        acts, as the inverse real FFT reads only the real
 *                        part of those bins.
 */
typedef enum {
  SPECTRE_GATE_REAL = 0,
  SPECTRE_GATE_LOGIT = 1,
  SPECTRE_GATE_COMPLEX = 2
} spectre_gate_kind;

/*
 * Where the norm sits and which norm it is (the *_ex entry points; the
 * others use POST).  Bit 0 is the order, bit 1 the norm:
 *  SPECTRE_NORM_POST: out = LayerNorm(x + y)   (section 2.2's pseudocode)
 *  SPECTRE_NORM_PRE:  out = x + LayerNorm(y)   (the order section 3.3 settles
 *                     on: the inverse FFT output is normalised, then added
 *                     to x), the same LayerNorm (eps 1e-5, biased variance,
 *                     gamma, beta) applied to y alone.
 *  SPECTRE_NORM_POST_RMS, SPECTRE_NORM_PRE_RMS: the same orders with
 *                     RMSNorm (section 3.3 allows RMSNorm or LayerNorm):
 *                     z / sqrt(mean_c(z^2) + 1e-5) * gamma + beta, no mean
 *                     subtracted (beta = 0 gives the textbook RMSNorm).
 */
typedef enum {
  SPECTRE_NORM_POST = 0,
  SPECTRE_NORM_PRE = 1,
  SPECTRE_NORM_POST_RMS = 2,
  SPECTRE_NORM_PRE_RMS = 3
} spectre_norm_order;

typedef enum {
  SPECTRE_OK = 0,
  SPECTRE_EINVAL = -1,       /* a null/misaligned pointer, bad size, dtype or keep_bins, aliasing */
  SPECTRE_EUNSUPPORTED = -2, /* a valid length/width this library does not implement */
  SPECTRE_ENOMEM = -3,       /* workspace or table allocation failed */
  SPECTRE_EHIP = -4          /* a HIP runtime call or kernel launch failed */
} spectre_status;

/*
 * The whole mix (see the top of this file): out = LayerNorm(x + y).
 * q, k, v, x: [B, L, H, D] dtype; gate: [H][L/2+1] f32; gamma, beta: [H*D] f32;
 * out: [B, L, H, D] dtype, must not overlap any input.
 * Returns SPECTRE_OK or an error code (nothing enqueued on error).
 */
int spectre_mix_fwd(const void* q, const void* k, const void* v, const void* x,
                    const float* gate, const float* gamma, const float* beta, void* out,
                    int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins, int dtype,
                    hipStream_t stream);

/*
 * spectre_mix_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, result and validation, but the call makes no
 * allocation at all -- no hipMalloc, no hipFree, no allocating library
 * routine.  Its workspace and tables live in a 64 MiB device array that the
 * library holds on every GPU it runs on until the process ends (its address
 * is looked up once per device, on the first call there).  Limits: plans of
 * one or two levels (L <= 65536 here, 2^a 3^b as for spectre_mix_fwd) whose
 * workspace and tables fit the 64 MiB (single-pass plans need 4 bytes per
 * element, B * L * H * D up to about 16 million; two-level plans 12 or 16
 * bytes per element, about 4 million); anything larger returns
 * SPECTRE_EUNSUPPORTED with
 * nothing enqueued.  All calls on one GPU share its array: calls that overlap
 * on one GPU (two streams, two threads) race and must be ordered by the
 * caller.  Every call writes all the array regions it reads.
 */
int spectre_mix_fwd_noalloc(const void* q, const void* k, const void* v, const void* x,
                            const float* gate, const float* gamma, const float* beta, void* out,
                            int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins,
                            int dtype, hipStream_t stream);

/*
 * The spectral part alone (same definition, stopped before the residual and
 * the norm): y [B, L, H, D] binary32, on the device, caller-owned, must not
 * overlap an input.  Used to check the transform directly, because the
 * LayerNorm hides a per-token scale error.
 */
int spectre_mix_y(const void* q, const void* k, const void* v, const float* gate, float* y,
                  int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins, int dtype,
                  hipStream_t stream);

/*
 * The mix with a chosen gate kind and norm order (spectre_gate_kind,
 * spectre_norm_order above); every other argument as for spectre_mix_fwd.
 * gate is [H][L/2+1] f32, or [H][L/2+1][2] f32 for SPECTRE_GATE_COMPLEX.
 * spectre_mix_fwd(...) is spectre_mix_fwd_ex(..., SPECTRE_GATE_REAL,
 * SPECTRE_NORM_POST, stream).  An unknown gate_kind or norm_order returns
 * SPECTRE_EINVAL (nothing enqueued).
 */
int spectre_mix_fwd_ex(const void* q, const void* k, const void* v, const void* x,
                       const float* gate, const float* gamma, const float* beta, void* out,
                       int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins,
                       int dtype, int gate_kind, int norm_order, hipStream_t stream);

/*
 * spectre_mix_y with a chosen gate kind (y does not depend on the norm order).
 */
int spectre_mix_y_ex(const void* q, const void* k, const void* v, const float* gate, float* y,
                     int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins, int dtype,
                     int gate_kind, hipStream_t stream);

/*
 * Chunked (blockwise) mix, for fft_len below L (the article's section 3.2:
 * an FFT inside fixed-size blocks, e.g. 4096 tokens, then one more
 * low-frequency interaction between the blocks, whose form the article
 * leaves open).  This library's reading:
 *   - each of the nb = L / fft_len blocks of fft_len tokens is mixed on its
 *     own: y_blk = the mix of the top of this file with length fft_len, gate
 *     [H][fft_len/2+1] and keep_bins <= fft_len/2 + 1;
 *   - the block means of q, k, v (nb values per column) are mixed by the same
 *     operation over the block axis: gate_blocks [H][nb/2+1] f32,
 *     keep_blocks <= nb/2 + 1; the result is added to every token of its
 *     block;
 *   - then out = LayerNorm(x + y) as for spectre_mix_fwd.
 * Shapes: fft_len a supported length (see above), L a multiple of it, nb
 * even with nb = 2^a * 3^b <= 2048, or nb in {3072, 4096} when
 * B * ceil(H*D / 8) <= 256 (else SPECTRE_EINVAL / EUNSUPPORTED).
 * Everything else (layouts, ownership, stream, errors) as spectre_mix_fwd.
 * The block means are the transform's bin 0 of each block, taken from the
 * forward pass; the block-axis mix runs between the transform and the norm.
 */
int spectre_mix_fwd_chunked(const void* q, const void* k, const void* v, const void* x,
                            const float* gate, const float* gate_blocks, const float* gamma,
                            const float* beta, void* out, int64_t B, int64_t H, int64_t L,
                            int64_t D, int64_t fft_len, int64_t keep_bins, int64_t keep_blocks,
                            int dtype, hipStream_t stream);

/* y of the chunked mix (binary32 [B, L, H, D]), the test hook's counterpart. */
int spectre_mix_y_chunked(const void* q, const void* k, const void* v, const float* gate,
                          const float* gate_blocks, float* y, int64_t B, int64_t H, int64_t L,
                          int64_t D, int64_t fft_len, int64_t keep_bins, int64_t keep_blocks,
                          int dtype, hipStream_t stream);

/*
 * The mix with the local branch (SPECTRE article, section 3.2's
 * use_local_branch and section 4.3: a sliding-window attention branch beside
 * the FFT branch, the two outputs added before the residual):
 *   out = LayerNorm_{H*D}(x + y + y_loc),
 * y the spectral mix of spectre_mix_fwd (real gate), and y_loc of head h at
 * token t the softmax over the keys j, t - win_left <= j <= t + win_right and
 * 0 <= j < L, of (q_t . k_j) / sqrt(D), applied to v_j (see
 * spectre_mix_local_attention).  Arguments, layout, ownership and errors as
 * spectre_mix_fwd, plus win_left, win_right >= 0 (else SPECTRE_EINVAL; a
 * window longer than the sequence is clipped to it), and D must be 16, 32,
 * 64 or 128 (else SPECTRE_EUNSUPPORTED).  The library's workspace is that
 * of spectre_mix_fwd (spectre_mix_workspace_bytes) plus 256 + 4 * B * L * H
 * * D bytes for y_loc, which the branch writes first and the LayerNorm pass
 * adds.
 */
int spectre_mix_fwd_local(const void* q, const void* k, const void* v, const void* x,
                          const float* gate, const float* gamma, const float* beta, void* out,
                          int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins,
                          int64_t win_left, int64_t win_right, int dtype, hipStream_t stream);

/*
 * spectre_mix_fwd_local with a chosen gate kind and norm order (as
 * spectre_mix_fwd_ex): SPECTRE_NORM_PRE gives out = x + LayerNorm(y + y_loc).
 * spectre_mix_fwd_local(...) is spectre_mix_fwd_local_ex(..., SPECTRE_GATE_REAL,
 * SPECTRE_NORM_POST, stream).  An unknown gate_kind or norm_order returns
 * SPECTRE_EINVAL (nothing enqueued).
 */
int spectre_mix_fwd_local_ex(const void* q, const void* k, const void* v, const void* x,
                             const float* gate, const float* gamma, const float* beta, void* out,
                             int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep_bins,
                             int64_t win_left, int64_t win_right, int dtype, int gate_kind,
                             int norm_order, hipStream_t stream);

/*
 * spectre_mix_fwd_local_ex with the two branches gated instead of summed
 * (SPECTRE article, section 4.3: the FFT and sliding-window outputs summed
 * or gated; read as a learned per-channel weight): the branch sum becomes
 *   g_c * y + (1 - g_c) * y_loc,   g_c = mix[c], c = h * D + d,
 * before the residual and the norm of norm_order.  mix: device, H * D
 * float32, 16-byte aligned, read only, owned by the caller; the values are
 * used as given (g = 1 keeps y alone, g = 0 y_loc alone; nothing is
 * clipped).  Every other argument, the workspace and the errors as
 * spectre_mix_fwd_local_ex; a null mix returns SPECTRE_EINVAL.
 */
int spectre_mix_fwd_local_gated(const void* q, const void* k, const void* v, const void* x,
                                const float* gate, const float* mix, const float* gamma,
                                const float* beta, void* out, int64_t B, int64_t H, int64_t L,
                                int64_t D, int64_t keep_bins, int64_t win_left, int64_t win_right,
                                int dtype, int gate_kind, int norm_order, hipStream_t stream);

/*
 * The local branch alone, the test hook of spectre_mix_fwd_local:
 * y[b, t, h, :] = sum_j p_j v[b, j, h, :], with p the softmax over the keys
 * j in [t - win_left, t + win_right] and [0, L) of (q[b,t,h,:] . k[b,j,h,:])
 * / sqrt(D).  q, k, v: [B, L, H, D] in `dtype` storage; y: binary32
 * [B, L, H, D], written whole, not overlapping q, k or v.  Any L >= 1;
 * D 16, 32, 64 or 128 (else SPECTRE_EUNSUPPORTED); pointers 16-byte
 * aligned, win_left, win_right >= 0 (else SPECTRE_EINVAL).  Uses no
 * workspace.  Asynchronous on `stream`.
 */
int spectre_mix_local_attention(const void* q, const void* k, const void* v, float* y, int64_t B,
                                int64_t H, int64_t L, int64_t D, int64_t win_left,
                                int64_t win_right, int dtype, hipStream_t stream);

/*
 * Device workspace bytes a spectre_mix_fwd call of this shape uses (0 if the
 * shape is invalid or unsupported): 4 bytes per element (y) for single-pass
 * plans (L <= 2048, and L = 3072, 4096 while B * ceil(H*D / 8) <= 256), 12 or
 * 16 per element for two-level plans (three spectra, and a fourth region when
 * the first pass writes its tiled layout), 24 for three-level plans, plus the
 * 4 * H * L-byte gate table of a multi-level plan whose LDS pass has 256 or
 * 1024 points.  Pure host arithmetic; no device call.
 */
size_t spectre_mix_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D, int dtype);

/* The same for a spectre_mix_fwd_ex call with this gate kind (a complex gate
 * doubles the gate table of multi-level plans). */
size_t spectre_mix_workspace_bytes_ex(int64_t B, int64_t H, int64_t L, int64_t D, int dtype,
                                      int gate_kind);

/*
 * Transform plan for length L, for inspection: the sequence length factors
 * as L = l1 * l2 * l3 (l1: first strided pass, l2: second strided pass, 1 if
 * absent; l3: the LDS-resident pass).  L = 3072 and 4096 report the single
 * pass (1, 1, L), which a call uses while B * ceil(H*D / 8) <= 256 (one
 * workgroup per 4 channel pairs, one round on the chip); larger calls at
 * those lengths use (L / 1024, 1, 1024).  Returns SPECTRE_OK or
 * SPECTRE_EUNSUPPORTED / SPECTRE_EINVAL.  No device call.
 */
int spectre_mix_plan(int64_t L, int64_t* l1, int64_t* l2, int64_t* l3);

/*
 * Frees the workspace and twiddle tables on every device the library has
 * used.  The caller must make sure no call's stream work is still pending.
 * Later calls recreate what they need.  Returns SPECTRE_OK or SPECTRE_EHIP.
 */
int spectre_mix_release(void);

/*
 * Per-kernel timing with HIP events (tracing).  After spectre_mix_trace_start,
 * each of the next `max_calls` calls to a computing entry point (spectre_mix_fwd,
 * spectre_mix_y and their _ex, _chunked and _local forms, and
 * spectre_mix_local_attention) also records a HIP event on its own stream
 * before its first kernel and after each kernel it enqueues; nothing
 * synchronises.  spectre_mix_trace_stop
 * waits for those events, stops tracing, and reports per position k of the
 * calls' launch sequence: total_ms[k] = summed duration over the traced
 * calls, names[k * name_len ...] = the kernel's short NUL-terminated name;
 * *n_kernels = kernels per call, *n_calls = calls traced.  Every traced call
 * must have the same shape (else SPECTRE_EINVAL).  Events are created by
 * start and destroyed by stop.  Returns SPECTRE_OK, SPECTRE_EINVAL or
 * SPECTRE_EHIP.
 */
int spectre_mix_trace_start(int max_calls);
int spectre_mix_trace_stop(int max_kernels, float* total_ms, int* n_kernels, int* n_calls,
                           char* names, int name_len);

/* Static, human-readable name of a status code (never NULL). */
const char* spectre_mix_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPECTRE_MIX_H */
