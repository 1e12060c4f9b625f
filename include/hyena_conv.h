/*
 * hyena_conv.h -- C ABI of the MI355X (gfx950) Hyena-SE / Hyena-MR operator
 * (forward, its backward, and both for filters of any length through the
 * FFT, further down)
 *
 *     y[b,t,d] = q[b,t,d] * sum_{s=0}^{min(t, l_h-1)} h[d / group_size, s] * k[b,t-s,d] * v[b,t-s,d]
 *
 * i.e. y = q (.) (h * (k (.) v)): a gated, grouped, depthwise causal FIR
 * convolution.  Sources (the StripedHyena 2 explainer pages):
 *   - page "04. hardware-aware convolution kernels", section 1, first
 *     equation: the causal FIR sum y_t = sum_j h_{t-j} x_j, h zero outside
 *     [0, l_h);
 *   - same page, section 3: the chunked (block-Toeplitz) form with chunk
 *     length l_b, Y_n = H0 X_n + H1 X_{n-1}, X_{-1} = 0;
 *   - same page, section 4, Algorithm 1: q gates the convolved chunk; k is
 *     loaded beside v and taken here as the pre-convolution gate, x = k (.) v;
 *   - same page, section 4, first bullet list: the channels of a group share
 *     one filter; channel d uses filter d / group_size.
 *
 * The library computes this with its own chunk length of 64 rows (the
 * value every workload here uses); the chunk length changes only the order
 * of the fp32 additions, never which terms are summed.  Filters may be up to
 * 2 * 64 = 128 taps long.  Where l_h > 65 the output chunk also reaches into
 * chunk n-2 (Y_n = H0 X_n + H1 X_{n-1} + H2 X_{n-2}); the library includes
 * that term, so the result is the convolution above for every l_h <= 128.
 *
 * Grouping: any group_size that divides D, down to one filter per channel.
 * When group_size is a multiple of 16 the channels of a group form the
 * matrix-core dimension (section 4 of the page above: one filter per group
 * lets the Toeplitz factors be shared across its channels).  Otherwise, for
 * filters longer than 8 taps, the work is laid out along the chunk direction
 * instead (same page, section 6): per channel, 16 consecutive 16-row
 * sub-chunks share each Toeplitz block; and for at most 8 taps each output's
 * few products are summed directly.  Off the 16-channel grouping D * element
 * size must be a multiple of 16 bytes (else HYENA_ERR_UNSUPPORTED).
 *
 * Layout (all row-major, no strides):
 *   q, k, v, out : [B, L, D], D contiguous.
 *   h            : [D / group_size, l_h], taps contiguous.
 * Precision:
 *   hyena_conv_fwd      : bf16 in, bf16 out.  k*v is formed in fp32 and
 *                         rounded once to bf16 (round to nearest even) as the
 *                         matrix-core operand; taps are bf16; sums are fp32;
 *                         the gated result is rounded once to bf16.  (The
 *                         direct sums off the grouping keep k*v in fp32.)
 *   hyena_conv_fwd_f32  : fp32 in, fp32 out, fp32 products and sums.
 *
 * Ownership and asynchrony: every pointer is a DEVICE pointer owned by the
 * caller.  The library allocates no device memory and keeps no state between
 * calls (apart from the fixed scratch array of hyena_conv_bwd_noalloc, below,
 * which is part of the loaded library).  Work is enqueued on
 * `stream` (a hipStream_t; NULL means the default stream) and the call
 * returns without waiting; the result is valid once the caller synchronises
 * that stream.  Calls on distinct streams are independent.
 *
 * Errors: integer status codes only -- nothing is printed, thrown or
 * aborted.  Argument checks run on the host before any HIP call, so a
 * rejected call touches no device state.  The output must not overlap any
 * input (other workgroups still read the inputs around an output row).
 */
#ifndef HYENA_CONV_H
#define HYENA_CONV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum hyena_status {
    HYENA_OK = 0,
    HYENA_ERR_NULL = -1,        /* a required pointer is NULL */
    HYENA_ERR_SHAPE = -2,       /* B, L or D negative, or sizes overflow */
    HYENA_ERR_GROUP = -3,       /* group_size < 1 or D % group_size != 0 */
    HYENA_ERR_FILTER_LEN = -4,  /* l_h outside [1, 128] */
    HYENA_ERR_ALIGN = -5,       /* q, k, v or out not 16-byte aligned, h not element aligned */
    HYENA_ERR_ALIAS = -6,       /* out overlaps an input (q, k, v, h, k_prev, v_prev) */
    HYENA_ERR_UNSUPPORTED = -7, /* a case outside the kernels' reach (see "Grouping"), or a shape they cannot address */
    HYENA_ERR_LAUNCH = -8,      /* the HIP runtime reported an error at launch */
    HYENA_ERR_DTYPE = -9,       /* unknown element-type code */
    HYENA_ERR_WORKSPACE = -10,  /* workspace missing or too small */
    HYENA_ERR_SCRATCH = -11     /* more scratch than hyena_conv_bwd_noalloc's fixed array holds */
};

enum hyena_dtype {
    HYENA_DTYPE_BF16 = 0,
    HYENA_DTYPE_F32 = 1
};

/* bf16 forward (see the top of this file).  B, L, D >= 0; an empty problem
 * (B == 0, L == 0 or D == 0) is a no-op that returns HYENA_OK. */
int hyena_conv_fwd(const void *q, const void *k, const void *v, const void *h,
                   int64_t B, int64_t L, int64_t D, int64_t group_size,
                   int64_t l_h, void *out, void *stream);

/* fp32 forward: same arguments and layout, every buffer float32. */
int hyena_conv_fwd_f32(const void *q, const void *k, const void *v,
                       const void *h, int64_t B, int64_t L, int64_t D,
                       int64_t group_size, int64_t l_h, void *out,
                       void *stream);

/* Either forward with an explicit work split: `dtype` is a hyena_dtype and
 * `span_chunks` is the number of consecutive 64-row chunks one workgroup
 * walks (0 = the library's choice, clamped to [1, ceil(L/64)]; when
 * group_size % 16 != 0 and l_h > 8 the walk is in 256-row blocks of 1, 2 or
 * 4, and the request is rounded to one of those).  The result
 * does not depend on `span_chunks`; it exists for tuning and for tests that
 * cover spans which do not divide the chunk count. */
int hyena_conv_fwd_ex(const void *q, const void *k, const void *v,
                      const void *h, int64_t B, int64_t L, int64_t D,
                      int64_t group_size, int64_t l_h, void *out, int dtype,
                      int64_t span_chunks, void *stream);

/* Forward of one shard of a longer sequence (context parallelism, point to
 * point): the history before row 0 of each batch row is not zero but the P
 * rows the caller passes, k_prev and v_prev ([B, P, D], same layout, dtype
 * and alignment as k, v; row P-1 immediately precedes row 0).  Only the last
 * l_h - 1 of them are read; if P < l_h - 1 the rows before those are zero.
 * P = 0 is hyena_conv_fwd_ex (k_prev, v_prev may then be NULL).  The result
 * equals rows [P, P + L) of the forward over the concatenated sequence
 * [prefix; q, k, v] (StripedHyena 2 explainer, page "01. overview", section
 * 5: context parallelism with point-to-point exchange; the operator itself is
 * the one at the top of this file).  out must not overlap k_prev or v_prev. */
int hyena_conv_fwd_halo(const void *q, const void *k, const void *v,
                        const void *h, const void *k_prev, const void *v_prev,
                        int64_t P, int64_t B, int64_t L, int64_t D,
                        int64_t group_size, int64_t l_h, void *out, int dtype,
                        int64_t span_chunks, void *stream);

/* Backward of the forward above for an upstream gradient dy ([B, L, D]):
 *     dq = dy (.) (h * (k (.) v)),         dz = dy (.) q,
 *     dx[t] = sum_{s < l_h, t+s < L} h[g, s] dz[t + s],
 *     dk = dx (.) v,   dv = dx (.) k,
 *     dh[g, s] = sum_{b, t, d in g} dz[b, t, d] x[b, t - s, d],  x = k (.) v.
 * (StripedHyena 2 explainer, page "04. hardware-aware convolution kernels",
 * section 7: the filter gradient is a global accumulation over positions,
 * computed in two back-to-back passes -- block-local partial gradients
 * written coalesced to `workspace`, then a vectorised reduction.)
 * dq, dk, dv are [B, L, D] in `dtype` (16-byte aligned); dh is float32
 * [D / group_size, l_h] (4-byte aligned) for either dtype.  Any of dq, dh
 * may be NULL (not computed); dk and dv are both given or both NULL.  With dh
 * the caller passes `workspace`, at least the size hyena_conv_bwd_workspace
 * reports (16-byte aligned, contents need not be initialised); it is
 * overwritten.  Outputs and workspace must not overlap the inputs or each
 * other.  bf16 precision as the forward: dz and x are rounded once to bf16
 * as matrix-core operands (off the 16-channel grouping with at most 8 taps,
 * the direct sums keep them in fp32), sums are fp32, outputs rounded once.
 * Results are the same run to run.  In bf16 a call with all four outputs reads q, k, v
 * and dy once; a call with fewer takes other kernels, whose fp32 sums may
 * group the same terms differently (dq, dh: last-place differences; fp32
 * calls give the same bits either way). */
int hyena_conv_bwd(const void *q, const void *k, const void *v, const void *h,
                   const void *dy, int64_t B, int64_t L, int64_t D,
                   int64_t group_size, int64_t l_h, void *dq, void *dk,
                   void *dv, float *dh, void *workspace,
                   int64_t workspace_bytes, int dtype, void *stream);

/* hyena_conv_bwd without a caller workspace and without any device
 * allocation, for callers that cannot allocate (code being captured into a
 * HIP graph, tight serving or training loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and bits as hyena_conv_bwd; the
 * partial filter gradients go to a fixed device array of the library,
 * hyena_conv_scratch_bytes() = 16 MiB, that every GPU the library runs on
 * holds until the process ends (its address is looked up on the first call
 * that needs it on a device).  A problem whose dh needs more than that
 * (hyena_conv_bwd_workspace reports the size: 16 MiB is B = 4, L = 32768,
 * D = 4096, 16-channel groups, l_h = 128) returns HYENA_ERR_SCRATCH before
 * any HIP call.  The array is shared by every call on one GPU and every
 * such call overwrites it before reading it: calls that may overlap in time
 * on one GPU (other streams, other host threads) race on it and must be
 * serialised by the caller.  Calls that do not compute dh do not touch it. */
int hyena_conv_bwd_noalloc(const void *q, const void *k, const void *v, const void *h,
                           const void *dy, int64_t B, int64_t L, int64_t D,
                           int64_t group_size, int64_t l_h, void *dq, void *dk,
                           void *dv, float *dh, int dtype, void *stream);

/* Size in bytes of hyena_conv_bwd_noalloc's fixed device array (16 MiB). */
int64_t hyena_conv_scratch_bytes(void);

/* Bytes of workspace hyena_conv_bwd needs to compute dh for these sizes
 * (written to *bytes_out).  Host only.  Returns a status. */
int hyena_conv_bwd_workspace(int64_t B, int64_t L, int64_t D,
                             int64_t group_size, int64_t l_h, int dtype,
                             int64_t *bytes_out);

/* Long-filter forward by FFT convolution, for filters of any length l_h >= 1
 * (Hyena-LI with a given filter).  Same operator, layout and dtypes as
 * hyena_conv_fwd_ex; taps past row L - 1 never contribute.  Computed as
 *     z = IFFT( FFT(h) * FFT(k (.) v) )[0, L),   y = q (.) z
 * with zero padding to N >= L + min(l_h, L) - 1 (a power of two, at most
 * 2^22), so the circular convolution equals the causal one (StripedHyena 2
 * explainer: page "01. overview", section 2, long convolutions through the
 * FFT in O(N log N); page "04. hardware-aware convolution kernels", section
 * 1, long filters are FFT-based).  The transforms are fp32 for both dtypes;
 * the error is that of an fp32 FFT (it is spread over the sequence, not
 * bounded per element by the direct sum's terms).  `workspace` (16-byte
 * aligned, at least hyena_conv_fwd_long_workspace bytes, contents need not be
 * initialised) receives the filter spectra and the transform work area.  D
 * must be even (channels are transformed in pairs), else
 * HYENA_ERR_UNSUPPORTED.  Inputs, output and workspace must not overlap.  The
 * filter spectra are recomputed on every call (hyena_conv_fwd_long_ex can
 * keep them). */
int hyena_conv_fwd_long(const void *q, const void *k, const void *v,
                        const void *h, int64_t B, int64_t L, int64_t D,
                        int64_t group_size, int64_t l_h, void *out, int dtype,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* hyena_conv_fwd_long with the filter spectra kept across calls.  The
 * spectra occupy the first 8 N G' bytes of `workspace` (N the transform
 * length, G' the filter count rounded up to even; they depend on L, l_h, D,
 * group_size and the filter, not on B).  reuse_spectra = 0: compute them
 * from h, as hyena_conv_fwd_long does; 1: the workspace already holds them,
 * left there by an earlier call on this stream with the same h, L, l_h, D,
 * group_size and dtype, and h is not read (it may be NULL).  The result has
 * the same bits either way.  With a workspace that does not hold them, the
 * output is meaningless (nothing is checked on the device).  Any other
 * reuse_spectra value returns HYENA_ERR_SHAPE. */
int hyena_conv_fwd_long_ex(const void *q, const void *k, const void *v,
                           const void *h, int64_t B, int64_t L, int64_t D,
                           int64_t group_size, int64_t l_h, void *out, int dtype,
                           void *workspace, int64_t workspace_bytes,
                           int reuse_spectra, void *stream);

/* Bytes of workspace hyena_conv_fwd_long needs (written to *bytes_out):
 * 8 N (max(B D/2, G'/2) + G'), N the transform length and G' the filter
 * count rounded up to even.  Host only.  Returns a status. */
int hyena_conv_fwd_long_workspace(int64_t B, int64_t L, int64_t D,
                                  int64_t group_size, int64_t l_h, int dtype,
                                  int64_t *bytes_out);

/* Backward of the long-filter forward, for filters of any length l_h >= 1:
 * the gradients of hyena_conv_bwd (same definitions, layouts, dtypes and
 * optional outputs: any of dq, dh may be NULL; dk and dv are both given or
 * both NULL; dh is float32 [D / group_size, l_h]), computed with the FFT
 * convolution of hyena_conv_fwd_long (StripedHyena 2 explainer: page
 * "01. overview", section 2, long convolutions in O(N log N); page
 * "04. hardware-aware convolution kernels", section 7, the filter gradient
 * is a global accumulation, here summed over channels and batch rows in the
 * frequency domain before one inverse transform per group).  With
 * N >= L + min(l_h, L) - 1 a power of two (at most 2^22):
 *     dq = dy (.) IFFT(H X),  dx = IFFT(conj(H) DZ),  dk = dx (.) v,
 *     dv = dx (.) k,  dh[g, s] = IFFT(sum_{b, c in g} DZ_c conj(X_c))[s],
 * x = k (.) v and dz = dy (.) q (exact in fp32 for bf16 inputs); dh is zero
 * at taps s >= L.  Transforms and sums are fp32 for both dtypes, with the
 * error of an fp32 FFT.  `workspace` (16-byte aligned, at least
 * hyena_conv_bwd_long_workspace bytes whenever an output is requested and
 * the problem has rows; contents need not be initialised) is overwritten.
 * D must be even, else HYENA_ERR_UNSUPPORTED.  Outputs and workspace must
 * not overlap the inputs or each other.  Results are the same run to run
 * (no atomics; fixed summation order). */
int hyena_conv_bwd_long(const void *q, const void *k, const void *v,
                        const void *h, const void *dy, int64_t B, int64_t L,
                        int64_t D, int64_t group_size, int64_t l_h, void *dq,
                        void *dk, void *dv, float *dh, int dtype,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* hyena_conv_bwd_long with the filter spectra kept in the workspace.  The
 * backward's workspace begins with the same 8 N G' bytes of filter spectra
 * as the forward's (they depend on L, l_h, D, group_size, dtype and the
 * filter, not on B): a hyena_conv_fwd_long_ex or hyena_conv_bwd_long(_ex)
 * call on this stream with the same h and sizes, given this workspace (at
 * least hyena_conv_bwd_long_workspace bytes, which covers the forward's),
 * leaves them there.  reuse_spectra = 0: compute them from h, as
 * hyena_conv_bwd_long does; 1: reuse them, h is not read (it may be NULL).
 * The results have the same bits either way; with a workspace that does not
 * hold them they are meaningless (nothing is checked on the device).  Any
 * other reuse_spectra value returns HYENA_ERR_SHAPE.  (For training: one
 * workspace kept from the forward to the backward saves the backward's
 * filter pass.) */
int hyena_conv_bwd_long_ex(const void *q, const void *k, const void *v,
                           const void *h, const void *dy, int64_t B, int64_t L,
                           int64_t D, int64_t group_size, int64_t l_h, void *dq,
                           void *dk, void *dv, float *dh, int dtype,
                           void *workspace, int64_t workspace_bytes,
                           int reuse_spectra, void *stream);

/* Bytes of workspace hyena_conv_bwd_long needs (written to *bytes_out):
 * 8 N (G' + B D + B T S) with N the transform length, G' the filter count
 * rounded up to even and T S the column tiles times the group slots per
 * tile of the filter gradient's partial sums (T S <= G + D).  Host only.
 * Returns a status. */
int hyena_conv_bwd_long_workspace(int64_t B, int64_t L, int64_t D,
                                  int64_t group_size, int64_t l_h, int dtype,
                                  int64_t *bytes_out);

/* The work split hyena_conv_fwd_ex would use: writes the chunks per
 * workgroup and the workgroup count.  Host only; runs the same argument
 * checks on the sizes (pointers are not inspected).  Returns a status. */
int hyena_conv_plan(int64_t B, int64_t L, int64_t D, int64_t group_size,
                    int64_t l_h, int dtype, int64_t span_chunks,
                    int64_t *span_out, int64_t *workgroups_out);

/* Static English text for a status code (never NULL). */
const char *hyena_conv_strerror(int status);

/* The library's chunk length l_b (64). */
int hyena_conv_block_len(void);

#ifdef __cplusplus
}
#endif

#endif /* HYENA_CONV_H */
