// Long-filter forward for MI355X (gfx950): y = q (.) (h * (k (.) v)) through
// FFT convolution, for filters of any length (Hyena-LI with a given filter).
//
// Method.  The long convolution is computed in O(N log N) with the fast
// Fourier transform (StripedHyena 2 explainer, page "01. overview", section
// 2 on the Hyena operator; page "04. hardware-aware convolution kernels",
// section 1: long filters go through the FFT, at low hardware utilisation).
// With N >= L + l_h - 1 (a power of two) the circular convolution of the
// zero-padded sequences equals the causal linear one on rows [0, L):
//     z = IFFT( FFT(h, N) * FFT(x, N) )[0, L),   x = k (.) v,   y = q (.) z.
//
// gfx950 mapping.  The [B, L, D] layout keeps channels contiguous, so the
// transforms run along the strided time axis, vectorised over channels, as a
// four-step FFT with N = N1 N2, t = t1 + N1 t2 and f = N2 f1 + f2:
//     X[N2 f1 + f2] = sum_t1 W_N1^(t1 f1) W_N^(t1 f2) sum_t2 x[t1 + N1 t2] W_N2^(t2 f2).
// Three kernels, each holding a transform of M <= 4096 points over a tile of
// P channel pairs in LDS:
//   1. fft_rows: per (batch, t1, pair tile): load the N2 rows t1 + N1 t2,
//      N2-point FFT, twiddle W_N^(t1 f2), write the workspace [B][N2][N1][pairs];
//   2. fft_cols: per (batch, column pair {f2, N2 - f2}, pair tile): N1-point
//      FFT of both columns, multiply by the filter spectra, inverse N1-point
//      FFT, twiddle W_N^(-t1 f2), write back in place (fft_col1: one column
//      at a time, when both channels of every pair share a filter);
//   3. fft_out: per (batch, t1, pair tile): inverse N2-point FFT, scale 1/N,
//      gate with q, store rows t1 + N1 t2 < L.
// Two real channels travel as one complex sequence (re = channel 2j, im =
// channel 2j + 1).  With P the packed spectrum, conj(P[-f]) recovers the two
// channel spectra, so one product serves both:
//     Z[f] = (H0 + H1)/2 P[f] + (H0 - H1)/2 conj(P[-f]),
// whose inverse transform is z0 + i z1 (H0, H1: the two channels' filter
// spectra; equal filters make the second term vanish).  The filter spectra
// come from the same two kernels run on the filters (pairs of filters,
// separated the same way; the filters first transposed to [taps][G'] fp32),
// once per call or kept across calls.
// Inner transforms are Stockham (self-sorting) in LDS, radix 16 (two radix-4
// levels in registers) per pass, with twiddles tabulated per workgroup;
// arithmetic is fp32 for both I/O types.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hyena_conv.h"

namespace {

constexpr int kFftThreads = 256;
// with at most 64 pairs per tile, 2P divides the thread count: a thread keeps
// one channel pair (and one column) across all its strided iterations
static_assert(kFftThreads % 128 == 0, "pair tiles of up to 64 pairs");
constexpr int kFftMaxLogN = 22;      // N <= 2^22
constexpr int kFftMaxLdsBytes = 160 * 1024;
// LDS per workgroup in complex values (pair tiles are sized to it)
#ifndef HYENA_FFT_BUDGET
#define HYENA_FFT_BUDGET 4096
#endif
constexpr int kFftBudget = HYENA_FFT_BUDGET;
#ifndef HYENA_FFT_COLS_BUDGET
#define HYENA_FFT_COLS_BUDGET HYENA_FFT_BUDGET
#endif
constexpr int kFftColsBudget = HYENA_FFT_COLS_BUDGET;  // the paired column kernels'
#ifndef HYENA_FFT_BWD_BUDGET
#define HYENA_FFT_BWD_BUDGET HYENA_FFT_BUDGET
#endif
constexpr int kFftBwdBudget = HYENA_FFT_BWD_BUDGET;  // the backward column kernels'
// The row, middle, output and single-column kernels transform in place (one
// LDS buffer: every value of a stage is read into registers, a barrier, then
// written), so their pair tiles are twice as wide as with two buffers.
#ifndef HYENA_FFT_INPLACE
#define HYENA_FFT_INPLACE 1
#endif
constexpr bool kFftInPlace = HYENA_FFT_INPLACE != 0;
// values per thread an in-place stage holds: M P <= kFftIpVals * kFftThreads
constexpr int kFftIpVals = kFftBudget / kFftThreads > 16 ? kFftBudget / kFftThreads : 16;

struct FftParams {
    const void *q, *k, *v, *h;
    void *y;
    void *y2;            // second output (the backward's dv), else unused
    float2 *ws;          // [nb][N2][N1][np] complex work area
    float2 *hs;          // [N2][N1][Gp] filter spectra
    float2 *part;        // backward: filter-gradient spectral partial sums, or null
    int32_t nb;          // backward: batch rows (a work area holds nb N np values)
    int32_t pb_log, pb_tiles, n_slots;  // backward: pairs per column tile (log2), those tiles, group slots per tile
    int32_t part_slot_major;  // backward: partials as part[b][tile][slot][f2][f1] (1) or [b][tile][f2][f1][slot] (0)
    int64_t L;           // rows of the input sequence (the filter pass: taps)
    int32_t D;           // channels (row pitch) of q, k, v, y
    int32_t np;          // channel pairs of this pass
    int32_t Gp;          // filters, rounded up to even
    int32_t G, group_size, l_h;
    int32_t N1, N2, log1, log2;
    int32_t N3, log3;    // third factor (1 for the two-level split)
    int32_t logP, n_tiles;  // pairs per workgroup (log2), pair tiles, of the kernel launched
};

__device__ inline float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ inline float2 cconj(float2 a) { return make_float2(a.x, -a.y); }

// exp(-2 pi i m / n) for 0 <= m < n, n a power of two <= 2^22 (2m/n is
// exact in fp32, and sincospif reduces it exactly).
__device__ inline float2 twiddle(int64_t m, int64_t n) {
    float s, c;
    sincospif((float)(2 * m) / (float)n, &s, &c);
    return make_float2(c, -s);
}

// Work item of this workgroup.  Workgroups are dispatched to the 8 XCDs in
// turn (workgroup i to XCD i mod 8), each with its own L2.  Consecutive work
// items (neighbouring pair tiles, which share 128-byte lines) are given to
// consecutive workgroups of one XCD: XCD x takes one contiguous run of items.
__device__ inline int xcd_item() {
    const int n = gridDim.x, bid = blockIdx.x;
    const int per = n >> 3, rem = n & 7, x = bid & 7;
    return x * per + min(x, rem) + (bid >> 3);
}

// Twiddle table tw[m] = exp(-2 pi i m / M), m < M.
__device__ inline void fill_twiddles(float2 *tw, int M) {
    for (int m = threadIdx.x; m < M; m += blockDim.x) tw[m] = twiddle(m, M);
}

// cos(2 pi m / 16), m taken mod 16: the constant twiddles of the
// in-register transforms (cos(pi/8), cos(pi/4), cos(3 pi/8), correctly
// rounded to fp32).
__host__ __device__ constexpr float cos16(int m) {
    constexpr float c1 = 0.923879532511286756f, c2 = 0.707106781186547524f, c3 = 0.382683432365089772f;
    switch (m & 15) {
    case 0: return 1.0f;
    case 1: return c1;
    case 2: return c2;
    case 3: return c3;
    case 4: return 0.0f;
    case 5: return -c3;
    case 6: return -c2;
    case 7: return -c1;
    case 8: return -1.0f;
    case 9: return -c1;
    case 10: return -c2;
    case 11: return -c3;
    case 12: return 0.0f;
    case 13: return c3;
    case 14: return c2;
    default: return c1;
    }
}
__host__ __device__ constexpr float sin16(int m) { return cos16(m - 4); }

// a W_R^m (INV: a W_R^-m) for a compile-time m, W_R = exp(-2 pi i / R),
// R dividing 16; multiples of a quarter turn cost no multiply.
template <int R, bool INV>
__device__ __forceinline__ float2 wconst(float2 a, int m) {
    const int e = (m * (16 / R)) & 15;
    if (e == 0) return a;
    if (e == 8) return make_float2(-a.x, -a.y);
    const bool neg_i = (e == 4) != INV;  // multiply by -i, else by +i (e = 4 or 12)
    if (e == 4 || e == 12) return neg_i ? make_float2(a.y, -a.x) : make_float2(-a.y, a.x);
    const float c = cos16(e), s = INV ? -sin16(e) : sin16(e);
    // a (c - i s)
    return make_float2(a.x * c + a.y * s, a.y * c - a.x * s);
}

// In-register DFT of R = 2, 4, 8 or 16 points (INV: the unscaled inverse).
template <int R, bool INV> __device__ __forceinline__ void dft(float2 *v);
template <> __device__ __forceinline__ void dft<2, false>(float2 *v) {
    const float2 a = v[0], b = v[1];
    v[0] = make_float2(a.x + b.x, a.y + b.y);
    v[1] = make_float2(a.x - b.x, a.y - b.y);
}
template <> __device__ __forceinline__ void dft<2, true>(float2 *v) { dft<2, false>(v); }
template <bool INV> __device__ __forceinline__ void dft4(float2 *v) {
    const float2 s02 = make_float2(v[0].x + v[2].x, v[0].y + v[2].y), d02 = make_float2(v[0].x - v[2].x, v[0].y - v[2].y);
    const float2 s13 = make_float2(v[1].x + v[3].x, v[1].y + v[3].y), d13 = make_float2(v[1].x - v[3].x, v[1].y - v[3].y);
    // W_4 d13 = -i d13 (forward), +i d13 (inverse)
    const float2 jd = INV ? make_float2(-d13.y, d13.x) : make_float2(d13.y, -d13.x);
    v[0] = make_float2(s02.x + s13.x, s02.y + s13.y);
    v[1] = make_float2(d02.x + jd.x, d02.y + jd.y);
    v[2] = make_float2(s02.x - s13.x, s02.y - s13.y);
    v[3] = make_float2(d02.x - jd.x, d02.y - jd.y);
}
template <> __device__ __forceinline__ void dft<4, false>(float2 *v) { dft4<false>(v); }
template <> __device__ __forceinline__ void dft<4, true>(float2 *v) { dft4<true>(v); }
// R = A B by one Cooley-Tukey split: with n = B n1 + n2 and k = k1 + A k2,
//     V[k1 + A k2] = sum_n2 W_B^(n2 k2) W_R^(n2 k1) sum_n1 v[B n1 + n2] W_A^(n1 k1).
template <int A, int B, bool INV> __device__ __forceinline__ void dft_split(float2 *v) {
    constexpr int R = A * B;
    float2 a[B][A];
#pragma unroll
    for (int n2 = 0; n2 < B; ++n2) {
        float2 t[A];
#pragma unroll
        for (int n1 = 0; n1 < A; ++n1) t[n1] = v[B * n1 + n2];
        dft<A, INV>(t);
#pragma unroll
        for (int k1 = 0; k1 < A; ++k1) a[n2][k1] = wconst<R, INV>(t[k1], n2 * k1);
    }
#pragma unroll
    for (int k1 = 0; k1 < A; ++k1) {
        float2 t[B];
#pragma unroll
        for (int n2 = 0; n2 < B; ++n2) t[n2] = a[n2][k1];
        dft<B, INV>(t);
#pragma unroll
        for (int k2 = 0; k2 < B; ++k2) v[k1 + A * k2] = t[k2];
    }
}
template <> __device__ __forceinline__ void dft<8, false>(float2 *v) { dft_split<4, 2, false>(v); }
template <> __device__ __forceinline__ void dft<8, true>(float2 *v) { dft_split<4, 2, true>(v); }
template <> __device__ __forceinline__ void dft<16, false>(float2 *v) { dft_split<4, 4, false>(v); }
template <> __device__ __forceinline__ void dft<16, true>(float2 *v) { dft_split<4, 4, true>(v); }

// One Stockham (self-sorting) stage of radix R on M points of P = 2^logP
// interleaved sequences (element j of sequence p at x[j P + p]): it combines
// R sub-transforms of Ns points into R Ns points.  For j < M/R, k = j mod Ns,
//     v_r = x[j + r M/R] W_(R Ns)^(r k),   V = DFT_R(v),
//     y[(j - k) R + k + r Ns] = V_r,
// with W conjugated (and DFT_R inverted) for the inverse transform.  tw[m] =
// W_M^m for m < M.
template <int R, bool INV>
__device__ __forceinline__ void fft_stage(const float2 *x, float2 *y, const float2 *tw, int M, int logP, int Ns,
                                          int logNs) {
    const int pmask = (1 << logP) - 1;
    const int n = (M / R) << logP;
    const int tstride = (M / R) >> logNs;  // W_(R Ns)^k = W_M^(k M / (R Ns))
    for (int i = threadIdx.x; i < n; i += kFftThreads) {
        const int j = i >> logP;
        const int p = i & pmask;
        const int k = j & (Ns - 1);
        float2 v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = x[i + r * n];
        if (Ns > 1) {
#pragma unroll
            for (int r = 1; r < R; ++r) {
                float2 w = tw[r * k * tstride];
                if (INV) w.y = -w.y;
                v[r] = cmul(v[r], w);
            }
        }
        dft<R, INV>(v);
        const int d = (j - k) * R + k;
#pragma unroll
        for (int r = 0; r < R; ++r) y[((d + r * Ns) << logP) + p] = v[r];
    }
}

// In-LDS M-point transform of P = 2^logP interleaved sequences: radix-16
// stages in registers while four or more bits of log2 M remain, then one of
// radix 8, 4 or 2.  Output in natural order; returns the buffer holding it.
// Callers synchronise before (x written) and the routine ends synchronised.
__device__ __forceinline__ float2 *lds_fft(float2 *x, float2 *y, const float2 *tw, int M, int logM, int logP,
                                         bool inverse) {
    int Ns = 1, logNs = 0;
    while (logNs < logM) {
        const int lr = logM - logNs >= 4 ? 4 : logM - logNs;
        if (inverse) {
            if (lr == 4) fft_stage<16, true>(x, y, tw, M, logP, Ns, logNs);
            else if (lr == 3) fft_stage<8, true>(x, y, tw, M, logP, Ns, logNs);
            else if (lr == 2) fft_stage<4, true>(x, y, tw, M, logP, Ns, logNs);
            else fft_stage<2, true>(x, y, tw, M, logP, Ns, logNs);
        } else {
            if (lr == 4) fft_stage<16, false>(x, y, tw, M, logP, Ns, logNs);
            else if (lr == 3) fft_stage<8, false>(x, y, tw, M, logP, Ns, logNs);
            else if (lr == 2) fft_stage<4, false>(x, y, tw, M, logP, Ns, logNs);
            else fft_stage<2, false>(x, y, tw, M, logP, Ns, logNs);
        }
        Ns <<= lr;
        logNs += lr;
        __syncthreads();
        float2 *t = x;
        x = y;
        y = t;
    }
    return x;
}

// One Stockham stage in place: the same butterflies as fft_stage, every
// value read into registers first (at most kFftIpVals per thread), then a
// barrier, then the writes.
template <int R, bool INV>
__device__ __forceinline__ void fft_stage_ip(float2 *x, const float2 *tw, int M, int logP, int Ns, int logNs) {
    constexpr int U = kFftIpVals / R > 0 ? kFftIpVals / R : 1;
    const int pmask = (1 << logP) - 1;
    const int n = (M / R) << logP;
    const int tstride = (M / R) >> logNs;
    float2 v[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        if (i >= n) continue;
        const int k = (i >> logP) & (Ns - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) v[u][r] = x[i + r * n];
        if (Ns > 1) {
#pragma unroll
            for (int r = 1; r < R; ++r) {
                float2 w = tw[r * k * tstride];
                if (INV) w.y = -w.y;
                v[u][r] = cmul(v[u][r], w);
            }
        }
        dft<R, INV>(v[u]);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        if (i >= n) continue;
        const int j = i >> logP, p = i & pmask, k = j & (Ns - 1);
        const int d = (j - k) * R + k;
#pragma unroll
        for (int r = 0; r < R; ++r) x[((d + r * Ns) << logP) + p] = v[u][r];
    }
    __syncthreads();
}

// lds_fft in place on x (M P <= kFftIpVals * kFftThreads); ends synchronised.
__device__ __forceinline__ void lds_fft_ip(float2 *x, const float2 *tw, int M, int logM, int logP, bool inverse) {
    int Ns = 1, logNs = 0;
    while (logNs < logM) {
        const int lr = logM - logNs >= 4 ? 4 : logM - logNs;
        if (inverse) {
            if (lr == 4) fft_stage_ip<16, true>(x, tw, M, logP, Ns, logNs);
            else if (lr == 3) fft_stage_ip<8, true>(x, tw, M, logP, Ns, logNs);
            else if (lr == 2) fft_stage_ip<4, true>(x, tw, M, logP, Ns, logNs);
            else fft_stage_ip<2, true>(x, tw, M, logP, Ns, logNs);
        } else {
            if (lr == 4) fft_stage_ip<16, false>(x, tw, M, logP, Ns, logNs);
            else if (lr == 3) fft_stage_ip<8, false>(x, tw, M, logP, Ns, logNs);
            else if (lr == 2) fft_stage_ip<4, false>(x, tw, M, logP, Ns, logNs);
            else fft_stage_ip<2, false>(x, tw, M, logP, Ns, logNs);
        }
        Ns <<= lr;
        logNs += lr;
    }
}

// The transform of the row-like kernels: in place on buf0 (buf1 unused), or
// ping-ponged between buf0 and buf1.  Returns the buffer holding the result.
__device__ __forceinline__ float2 *lds_fft1(float2 *buf0, float2 *buf1, const float2 *tw, int M, int logM, int logP,
                                          bool inverse) {
    if constexpr (kFftInPlace) {
        lds_fft_ip(buf0, tw, M, logM, logP, inverse);
        return buf0;
    } else {
        return lds_fft(buf0, buf1, tw, M, logM, logP, inverse);
    }
}
constexpr int kRowBufs = kFftInPlace ? 1 : 2;  // LDS buffers of the row-like kernels

// Register-fed transforms.  With a full tile (M P = 16 kFftThreads values)
// and a radix-16 first stage, that stage's butterfly of thread tid takes
// x[tid + r kFftThreads], r < 16: the same 16 values the thread would stage
// to LDS, so they go from the global loads straight into the butterfly.  The
// last stage's results stay in registers too: with R its radix, U = 16 / R
// and Ns = M / R, value e = u R + r of the thread is output f = j + r Ns of
// pair tid mod P, where j = (tid + u kFftThreads) >> logP.  Only the stages
// in between pass through LDS.  The butterflies and twiddles are those of
// lds_fft_ip; results can differ from it in the last bit, since the compiler
// contracts the complex products into fused multiply-adds differently.
// The 16 outputs of a thread are, for every R, the inputs of its first
// stage in the next transform of the same tile (f = tid >> logP + (M / 16) r'
// with r' = u + r U), so a forward and an inverse transform chain in
// registers (fft_reg_perm).
constexpr int kFftRegVals = 16;
static_assert(kFftIpVals >= kFftRegVals, "the in-place stages hold a full tile per thread");

// (32 to 256 points: the first stage and the last, nothing in between)
__device__ inline bool fft_reg_ok(int logM, int logP) {
    return logM >= 5 && logM <= 8 && (1 << (logM + logP)) == kFftRegVals * kFftThreads;
}
// log2 of the last stage's radix: radix-16 stages while more than four bits remain
__host__ __device__ inline int fft_last_log(int logM) { return logM - 4 * ((logM - 1) / 4); }
// output index of value e of this thread after the last stage of radix 2^lr
__device__ inline int fft_reg_out(int e, int lr, int logM, int logP) {
    return ((threadIdx.x + (e >> lr) * kFftThreads) >> logP) + (e & ((1 << lr) - 1)) * (1 << (logM - lr));
}

// First stage (radix 16, no twiddles) from v[r] = x[tid + r kFftThreads];
// writes its outputs to x.  The caller synchronises afterwards.
template <bool INV>
__device__ __forceinline__ void fft_reg_first(float2 *x, int logP, float2 (&v)[kFftRegVals]) {
    dft<16, INV>(v);
    const int j = threadIdx.x >> logP, p = threadIdx.x & ((1 << logP) - 1);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[((16 * j + r) << logP) + p] = v[r];
}

// The last stage of radix R (Ns = M / R) from x into v[u R + r].
template <int R, bool INV>
__device__ __forceinline__ void fft_reg_last(const float2 *x, const float2 *tw, int logP, int Ns,
                                             float2 (&v)[kFftRegVals]) {
    constexpr int U = kFftRegVals / R;
    const int n = Ns << logP;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        const int j = i >> logP;  // < Ns: also the twiddle index
        float2 t[R];
#pragma unroll
        for (int r = 0; r < R; ++r) t[r] = x[i + r * n];
#pragma unroll
        for (int r = 1; r < R; ++r) {
            float2 w = tw[r * j];
            if (INV) w.y = -w.y;
            t[r] = cmul(t[r], w);
        }
        dft<R, INV>(t);
#pragma unroll
        for (int r = 0; r < R; ++r) v[u * R + r] = t[r];
    }
}

// The second and last stage (x synchronised on entry; M = 16 2^lr) into v.
// Returns without a barrier after its reads of x.
template <bool INV>
__device__ __forceinline__ void fft_reg_rest(float2 *x, const float2 *tw, int logM, int logP,
                                             float2 (&v)[kFftRegVals]) {
    const int lr = logM - 4;
    if (lr == 4) fft_reg_last<16, INV>(x, tw, logP, 16, v);
    else if (lr == 3) fft_reg_last<8, INV>(x, tw, logP, 16, v);
    else if (lr == 2) fft_reg_last<4, INV>(x, tw, logP, 16, v);
    else fft_reg_last<2, INV>(x, tw, logP, 16, v);
}

// Last-stage outputs (v[u R + r]) reordered as first-stage inputs of the
// same tile (v[u + r U]).
template <int R> __device__ __forceinline__ void fft_reg_perm(float2 (&v)[kFftRegVals]) {
    constexpr int U = kFftRegVals / R;
    float2 t[kFftRegVals];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) t[u + r * U] = v[u * R + r];
#pragma unroll
    for (int e = 0; e < kFftRegVals; ++e) v[e] = t[e];
}

// Global -> LDS staging of n values, NB per thread at a time: the loads of a
// batch are issued together (indices clamped into range, so none is
// conditional) and waited for once.  Sixteen at a time when a thread stages
// at least that many (all of a 4096-value tile in one batch), else eight.
#ifndef HYENA_FFT_BATCH
#define HYENA_FFT_BATCH 8
#endif
constexpr int kBatch = HYENA_FFT_BATCH;  // also the batch of the filter-spectrum loads
// Filter counts up to this read h [G][l_h] directly in the filter pass (one
// element per filter row; the rows are shared through L2); more filters are
// first transposed to fp32 [taps][G'], so each pair is one 8-byte read.
#ifndef HYENA_FFT_DIRECT_FILTERS
#define HYENA_FFT_DIRECT_FILTERS 512
#endif
constexpr int64_t kFftDirectFilters = HYENA_FFT_DIRECT_FILTERS;
template <int NB, typename Load>
__device__ inline void stage_in_nb(float2 *dst, int n, Load load) {
    for (int base = 0; base < n; base += NB * kFftThreads) {
        float2 r[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) r[u] = load(min(base + u * kFftThreads + (int)threadIdx.x, n - 1));
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int i = base + u * kFftThreads + (int)threadIdx.x;
            if (i < n) dst[i] = r[u];
        }
    }
}
template <typename Load>
__device__ inline void stage_in(float2 *dst, int n, Load load) {
    if (n >= 16 * kFftThreads)
        stage_in_nb<16>(dst, n, load);
    else
        stage_in_nb<kBatch>(dst, n, load);
}

// Input pair j at row t, zero past the end of the sequence or the pairs:
// (x[2j], x[2j+1]) with x = k v (SRC = 0, batch row b), or (h[2j][t],
// h[2j+1][t]) (the filters; zero for a filter past the last) from the
// transposed fp32 copy (SRC = 1) or from h [G][l_h] itself (SRC = 2: one
// element per filter row).  The loads always go to a valid address (row 0,
// pair 0 when out of range) and the value is then replaced by zero.
template <bool F32, int SRC>
__device__ inline float2 load_pair(const FftParams &p, int b, int64_t t, int j) {
    const bool ok = t < p.L && j < p.np;
    const int64_t tc = ok ? t : 0;
    const int jc = ok ? j : 0;
    float a, c;
    if constexpr (SRC == 0) {
        const size_t o = ((size_t)b * (size_t)p.L + (size_t)tc) * (size_t)p.D + 2 * (size_t)jc;
        if constexpr (F32) {
            const float2 kk = *(const float2 *)((const float *)p.k + o);
            const float2 vv = *(const float2 *)((const float *)p.v + o);
            a = kk.x * vv.x;
            c = kk.y * vv.y;
        } else {
            const uint32_t kk = *(const uint32_t *)((const uint16_t *)p.k + o);
            const uint32_t vv = *(const uint32_t *)((const uint16_t *)p.v + o);
            a = __uint_as_float(kk << 16) * __uint_as_float(vv << 16);
            c = __uint_as_float(kk & 0xffff0000u) * __uint_as_float(vv & 0xffff0000u);
        }
    } else if constexpr (SRC == 1) {
        // the filters transposed to fp32 [taps][Gp] (fft_filter_transpose_kernel)
        const float2 hh = *(const float2 *)((const float *)p.h + (size_t)tc * p.Gp + 2 * (size_t)jc);
        a = hh.x;
        c = hh.y;
    } else {
        // the filters as given, [G][l_h]; filter 2j + 1 = G (odd G) is zero
        const bool two = 2 * jc + 1 < p.G;
        const size_t o0 = (size_t)(2 * jc) * (size_t)p.l_h + (size_t)tc, o1 = two ? o0 + (size_t)p.l_h : o0;
        if constexpr (F32) {
            a = ((const float *)p.h)[o0];
            c = ((const float *)p.h)[o1];
        } else {
            a = __uint_as_float((uint32_t)((const uint16_t *)p.h)[o0] << 16);
            c = __uint_as_float((uint32_t)((const uint16_t *)p.h)[o1] << 16);
        }
        c = two ? c : 0.0f;
    }
    return ok ? make_float2(a, c) : make_float2(0.0f, 0.0f);
}

// The filters h [G][l_h] (dtype) -> hT [taps][Gp] fp32, filter Gp - 1 zero
// when G is odd: the filter pass of the row kernel then reads a pair of
// filters at one tap as 8 contiguous bytes, as it reads channel pairs of the
// sequence.  64 x 64 tiles through LDS; reads run along taps, writes along
// filters.
template <bool F32>
__global__ __launch_bounds__(256) void fft_filter_transpose_kernel(const void *h, float *hT, int G, int Gp, int l_h,
                                                                  int taps, int n_tblk) {
    __shared__ float tile[64][65];
    const int t0 = (int)(blockIdx.x % n_tblk) * 64, g0 = (int)(blockIdx.x / n_tblk) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    // all 16 loads of a thread in flight together
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int g = g0 + ty + 4 * u, t = t0 + tx;
        v[u] = 0.0f;
        if (g < G && t < taps) {
            const size_t o = (size_t)g * l_h + t;
            v[u] = F32 ? ((const float *)h)[o] : __uint_as_float((uint32_t)((const uint16_t *)h)[o] << 16);
        }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) tile[ty + 4 * u][tx] = v[u];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int r = ty + 4 * u;
        const int t = t0 + r, g = g0 + tx;
        if (t < taps && g < Gp) hT[(size_t)t * Gp + g] = tile[tx][r];
    }
}

// Kernel 1: forward transform along t2 for one t1, then the twiddle.
// LDS (dynamic): one buffer (in place) of N2 P values, the N2 inner twiddles and the
// N2 inter-step twiddles W_N^(t1 f2) of this t1.
template <bool F32, int SRC, bool REG>
__global__ __launch_bounds__(kFftThreads) void fft_rows_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int t1 = (item / p.n_tiles) % p.N1;
    const int b = item / (p.n_tiles * p.N1);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1, N2 = p.N2;
    const int NP = N2 << logP;
    const int64_t N = (int64_t)N1 * N2;
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + kRowBufs * NP, *wt = tw + N2;
    if constexpr (REG) {
        // full tile: loads into the first stage, the last stage into the stores
        if (!fft_reg_ok(p.log2, logP)) return;  // the host launches this form only for full tiles
        const int j = (tile << logP) + (threadIdx.x & pmask);
        float2 v[kFftRegVals];
#pragma unroll
        for (int u = 0; u < kFftRegVals; ++u)
            v[u] = load_pair<F32, SRC>(p, b, t1 + (int64_t)N1 * ((threadIdx.x + u * kFftThreads) >> logP), j);
        fill_twiddles(tw, N2);
        for (int f2 = threadIdx.x; f2 < N2; f2 += kFftThreads) wt[f2] = twiddle(((int64_t)t1 * f2) & (N - 1), N);
        fft_reg_first<false>(buf0, logP, v);
        __syncthreads();
        fft_reg_rest<false>(buf0, tw, p.log2, logP, v);
        if (j < p.np) {
            const int lr = fft_last_log(p.log2);
#pragma unroll
            for (int e = 0; e < kFftRegVals; ++e) {
                const int f2 = fft_reg_out(e, lr, p.log2, logP);
                p.ws[(((int64_t)b * N2 + f2) * N1 + t1) * p.np + j] = cmul(v[e], wt[f2]);
            }
        }
        return;
    }
    stage_in(buf0, NP, [&](int i) {
        return load_pair<F32, SRC>(p, b, t1 + (int64_t)N1 * (i >> logP), (tile << logP) + (i & pmask));
    });
    fill_twiddles(tw, N2);
    for (int f2 = threadIdx.x; f2 < N2; f2 += kFftThreads) wt[f2] = twiddle(((int64_t)t1 * f2) & (N - 1), N);
    __syncthreads();
    const float2 *X = lds_fft1(buf0, buf1, tw, N2, p.log2, logP, false);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int f2 = i >> logP;
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        p.ws[(((int64_t)b * N2 + f2) * N1 + t1) * p.np + j] = cmul(X[i], wt[f2]);
    }
}

// Kernel 2: transforms along t1 for the column pair {f2, N2 - f2}.
// MODE 0 (filters): separate each pair's packed spectrum into the two
// filters' spectra and store them in hs.  MODE 1 (sequence): multiply by the
// filter spectra, inverse transform along f1, twiddle, store in place.
// The two columns are interleaved in LDS -- element (t1, col, pair) at
// (2 t1 + col) P + pair -- so one transform of 2P sequences covers both.  A
// self-paired column (f2 = 0 or N2/2) is staged twice and stored once.
// In place (one buffer) the products go to registers first: each reads a
// partner value another thread may overwrite.
// LDS (dynamic): one (in place) or two buffers of 2 N1 P values, the N1
// inner twiddles and, per column, the N1 inter-step twiddles W_N^(-t1 f2).
template <int MODE>
__global__ __launch_bounds__(kFftThreads) void fft_cols_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int N2 = p.N2 * p.N3;  // columns (M of the three-level split)
    const int c = (item / p.n_tiles) % (N2 / 2 + 1);
    const int b = item / (p.n_tiles * (N2 / 2 + 1));
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1;
    const int lP2 = logP + 1;
    const int NP2 = N1 << lP2;
    const int64_t N = (int64_t)N1 * N2;
    const int fa = c, fb = (N2 - c) & (N2 - 1);
    const bool self = fa == fb;
    // work-area position of column f: (f mod N3) N2 + f / N3 (the identity
    // for the two-level split), so the middle passes work in place
    auto cpos = [&](int f) -> int64_t { return (int64_t)(f & (p.N3 - 1)) * p.N2 + (f >> p.log3); };
    float2 *bufA = lds, *bufB = lds + NP2, *tw = lds + kRowBufs * NP2;
    float2 *wt[2] = {tw + N1, tw + 2 * N1};
    stage_in(bufA, NP2, [&](int i) {
        const int col = (i >> logP) & 1;
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[(((int64_t)b * N2 + cpos(col ? fb : fa)) * N1 + (i >> lP2)) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N1);
    if constexpr (MODE == 1) {
        for (int i = threadIdx.x; i < 2 * N1; i += kFftThreads) {
            const int col = i >= N1 ? 1 : 0, t1 = i - col * N1;
            wt[col][t1] = cconj(twiddle(((int64_t)t1 * (col ? fb : fa)) & (N - 1), N));
        }
    }
    __syncthreads();
    float2 *S = lds_fft1(bufA, bufB, tw, N1, p.log1, lP2, false);
    float2 *Z = kFftInPlace ? S : (S == bufA ? bufB : bufA);
    // 2P divides the thread count, so a thread always has the same column
    // and channel pair: its filter spectra rows are fixed
    const int my_col = (threadIdx.x >> logP) & 1, my_pp = threadIdx.x & pmask;
    const int my_f2 = my_col ? fb : fa;
    const int my_j = (tile << logP) + my_pp;
    const int jc = min(my_j, p.np - 1);
    const float2 *hrow0 = p.hs + (size_t)my_f2 * N1 * p.Gp + (2 * jc) / p.group_size;
    const float2 *hrow1 = p.hs + (size_t)my_f2 * N1 * p.Gp + (2 * jc + 1) / p.group_size;
    // (in place) this thread's products, value u at i = tid + u kFftThreads
    float2 zr[kFftInPlace && MODE == 1 ? kFftIpVals : 1];
#pragma unroll
    for (int ub = 0; ub < kFftIpVals; ub += kBatch) {
        const int base = ub * kFftThreads;
        if (base >= NP2) break;
        float2 h0[kBatch], h1[kBatch];
        if constexpr (MODE == 1) {
            // filter spectra of this batch, all loads in flight together
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int f1 = min(base + u * kFftThreads + (int)threadIdx.x, NP2 - 1) >> lP2;
                h0[u] = hrow0[(size_t)f1 * p.Gp];
                h1[u] = hrow1[(size_t)f1 * p.Gp];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = base + u * kFftThreads + (int)threadIdx.x;
            if (i >= NP2) continue;
            const int f1 = i >> lP2, col = my_col, pp = my_pp;
            const int f2 = my_f2;
            const int j = my_j;
            // -(N2 f1 + f2) mod N = N2 f1m + (N2 - f2) mod N2: the other column
            const int f1m = (N1 - f1 - (f2 > 0 ? 1 : 0)) & (N1 - 1);
            const float2 a = S[i];
            const float2 m = cconj(S[(((f1m << 1) | (col ^ 1)) << logP) + pp]);
            if constexpr (MODE == 0) {
                // filters 2j and 2j + 1: (a + m)/2 and (a - m)/(2i)
                if (j < p.np && !(self && col)) {
                    const size_t o = ((size_t)f2 * N1 + f1) * p.Gp + 2 * (size_t)j;
                    p.hs[o] = make_float2(0.5f * (a.x + m.x), 0.5f * (a.y + m.y));
                    p.hs[o + 1] = make_float2(0.5f * (a.y - m.y), -0.5f * (a.x - m.x));
                }
            } else {
                // (H0 + H1)/2 P[f] + (H0 - H1)/2 conj(P[-f])
                const float2 sm = make_float2(0.5f * (h0[u].x + h1[u].x), 0.5f * (h0[u].y + h1[u].y));
                const float2 df = make_float2(0.5f * (h0[u].x - h1[u].x), 0.5f * (h0[u].y - h1[u].y));
                const float2 pu = cmul(sm, a), pv = cmul(df, m);
                const float2 zv = j < p.np ? make_float2(pu.x + pv.x, pu.y + pv.y) : make_float2(0.0f, 0.0f);
                if constexpr (kFftInPlace)
                    zr[ub + u] = zv;
                else
                    Z[i] = zv;
            }
        }
    }
    if constexpr (MODE == 1) {
        __syncthreads();
        if constexpr (kFftInPlace) {
#pragma unroll
            for (int u = 0; u < kFftIpVals; ++u) {
                const int i = threadIdx.x + u * kFftThreads;
                if (i < NP2) Z[i] = zr[u];
            }
            __syncthreads();
        }
        const float2 *U = lds_fft1(Z, S, tw, N1, p.log1, lP2, true);
        for (int i = threadIdx.x; i < NP2; i += kFftThreads) {
            const int t1 = i >> lP2, col = (i >> logP) & 1;
            const int j = (tile << logP) + (i & pmask);
            if (j >= p.np || (self && col)) continue;
            p.ws[(((int64_t)b * N2 + cpos(col ? fb : fa)) * N1 + t1) * p.np + j] = cmul(U[i], wt[col][t1]);
        }
    }
}

// Kernel 2, single-column form, for a sequence whose channel pairs each lie
// inside one group (even group sizes): H0 = H1, so Z = H P[f] and a column
// needs no partner.  Per (batch, column f2, pair tile): N1-point FFT, the
// product with the group's filter spectrum, inverse N1-point FFT, twiddle
// W_N^(-t1 f2), store in place.  Half the LDS of the paired form per pair,
// so tiles are twice as wide (whole 128-byte work-area segments) and each
// point reads one filter spectrum value.
// LDS (dynamic): one buffer (in place) of N1 P values, the N1 inner twiddles and the N1
// inter-step twiddles.
// LR > 0: the register-fed form for full tiles whose last stage has radix 2^LR.
template <int LR>
__global__ __launch_bounds__(kFftThreads) void fft_col1_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int M = p.N2 * p.N3;  // columns
    const int f2 = (item / p.n_tiles) % M;
    const int b = item / (p.n_tiles * M);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1;
    const int NP = N1 << logP;
    const int64_t N = (int64_t)N1 * M;
    // work-area row of (f2, t1 = 0): column position as in the paired form
    const int64_t col0 = ((int64_t)b * M + (int64_t)(f2 & (p.N3 - 1)) * p.N2 + (f2 >> p.log3)) * N1;
    float2 *bufA = lds, *bufB = lds + NP, *tw = lds + kRowBufs * NP, *wt = tw + N1;
    // P divides the thread count, so a thread always has the same pair and
    // its filter spectrum row is fixed; its spectrum values (value u of the
    // thread: i = tid + u kFftThreads, NP <= kFftIpVals kFftThreads) are
    // loaded before the transform, to hide their latency behind it
    const int my_j = (tile << logP) + (threadIdx.x & pmask);
    const int jc = min(my_j, p.np - 1);
    const float2 *hrow = p.hs + (size_t)f2 * N1 * p.Gp + (2 * jc) / p.group_size;
    if constexpr (LR > 0) {
        // full tile: loads into the forward's first stage, its last stage
        // into the products and the inverse's first stage, the inverse's
        // last stage into the stores
        if (!fft_reg_ok(p.log1, logP) || fft_last_log(p.log1) != LR) return;  // the host's choice
        const bool ok = my_j < p.np;
        constexpr int lr = LR;
        // the filter spectra of this thread's frequencies, in flight during the forward transform
        float2 hr[kFftRegVals], v[kFftRegVals];
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e) hr[e] = hrow[(size_t)fft_reg_out(e, lr, p.log1, logP) * p.Gp];
#pragma unroll
        for (int u = 0; u < kFftRegVals; ++u) {
            const float2 x = p.ws[(col0 + ((threadIdx.x + u * kFftThreads) >> logP)) * p.np + (ok ? my_j : 0)];
            v[u] = ok ? x : make_float2(0.0f, 0.0f);
        }
        fill_twiddles(tw, N1);
        for (int t1 = threadIdx.x; t1 < N1; t1 += kFftThreads)
            wt[t1] = cconj(twiddle(((int64_t)t1 * f2) & (N - 1), N));
        fft_reg_first<false>(bufA, logP, v);
        __syncthreads();
        fft_reg_last<1 << LR, false>(bufA, tw, logP, 16, v);
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e) v[e] = ok ? cmul(hr[e], v[e]) : make_float2(0.0f, 0.0f);
        fft_reg_perm<1 << LR>(v);
        __syncthreads();  // every thread's last-stage reads are done
        fft_reg_first<true>(bufA, logP, v);
        __syncthreads();
        fft_reg_last<1 << LR, true>(bufA, tw, logP, 16, v);
        if (ok) {
#pragma unroll
            for (int e = 0; e < kFftRegVals; ++e) {
                const int t1 = fft_reg_out(e, lr, p.log1, logP);
                p.ws[(col0 + t1) * p.np + my_j] = cmul(v[e], wt[t1]);
            }
        }
        return;
    }
    float2 hh[kFftIpVals];
#pragma unroll
    for (int u = 0; u < kFftIpVals; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        if (i < NP) hh[u] = hrow[(size_t)(i >> logP) * p.Gp];
    }
    stage_in(bufA, NP, [&](int i) {
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[(col0 + (i >> logP)) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N1);
    for (int t1 = threadIdx.x; t1 < N1; t1 += kFftThreads)
        wt[t1] = cconj(twiddle(((int64_t)t1 * f2) & (N - 1), N));
    __syncthreads();
    float2 *S = lds_fft1(bufA, bufB, tw, N1, p.log1, logP, false);
    // the product goes to the other buffer, or (in place) over S: each
    // thread rewrites only the values it reads
    float2 *Z = kFftInPlace ? S : (S == bufA ? bufB : bufA);
#pragma unroll
    for (int u = 0; u < kFftIpVals; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        if (i < NP) Z[i] = my_j < p.np ? cmul(hh[u], S[i]) : make_float2(0.0f, 0.0f);
    }
    __syncthreads();
    const float2 *U = lds_fft1(Z, S, tw, N1, p.log1, logP, true);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        const int t1 = i >> logP;
        p.ws[(col0 + t1) * p.np + j] = cmul(U[i], wt[t1]);
    }
}

// Backward column kernel.  The work area holds two transforms side by side:
// x = k v (the first nb N np values) and dz = dy q (the next).  Per (batch,
// column pair {f2, M - f2}, pair tile): the N1-point transforms of both
// columns of both, then per frequency f, with a = P[f] and m = conj(P[-f]) of
// a packed pair spectrum and H0, H1 its two channels' filter spectra,
//     Z  = (H0 + H1)/2 a_x  + (H0 - H1)/2 m_x          (z = h * x, for dq)
//     DX = conj((H0 + H1)/2) a_dz + conj((H0 - H1)/2) m_dz   (dx, for dk, dv)
// since dx[t] = sum_s h[s] dz[t + s] is the correlation with h, whose
// spectrum is conj(H) DZ.  Both are transformed back along f1, twiddled and
// stored in place, as in the forward.  With `part` set it also writes the
// filter gradient's spectral partial sums: dh[g, s] = sum_{b, c in g} (dz_c
// correlated with x_c)[s], whose spectrum is sum DZ_c conj(X_c), the channel
// spectra separated as X_0 = (a + m)/2, X_1 = (a - m)/(2i):
//     channel 2j: (a_dz + m_dz) conj(a_x + m_x) / 4,
//     channel 2j + 1: (a_dz - m_dz) conj(a_x - m_x) / 4,
// summed over the tile's channels of each group into
// part[b][tile][f2][f1][slot], slot = group - first group of the tile
// (the single-column form: part[b][tile][slot][f2][f1]).
// LDS (dynamic): one buffer (in place) of 4 N1 P values -- element (t1, src, col,
// pair) at ((2 t1 + src) 2 + col) P + pair -- the N1 inner twiddles and,
// per column, the N1 inter-step twiddles W_N^(-t1 f2).
__global__ __launch_bounds__(kFftThreads) void fft_bwd_cols_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int M = p.N2 * p.N3;  // columns
    const int c = (item / p.n_tiles) % (M / 2 + 1);
    const int b = item / (p.n_tiles * (M / 2 + 1));
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1;
    const int lP2 = logP + 1, lS = logP + 2;
    const int NS = N1 << lS;
    const int sdz = 1 << lP2;  // from an x sequence to the dz sequence of the same column and pair
    const int64_t N = (int64_t)N1 * M;
    const int64_t area = (int64_t)p.nb * N * p.np;
    const int fa = c, fb = (M - c) & (M - 1);
    const bool self = fa == fb;
    auto cpos = [&](int f) -> int64_t { return (int64_t)(f & (p.N3 - 1)) * p.N2 + (f >> p.log3); };
    auto wpos = [&](int src, int col, int t1, int j) -> int64_t {
        return src * area + (((int64_t)b * M + cpos(col ? fb : fa)) * N1 + t1) * p.np + j;
    };
    float2 *bufA = lds, *bufB = lds + NS, *tw = lds + kRowBufs * NS;
    float2 *wt[2] = {tw + N1, tw + 2 * N1};
    stage_in(bufA, NS, [&](int i) {
        const int col = (i >> logP) & 1, src = (i >> lP2) & 1;
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[wpos(src, col, i >> lS, ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N1);
    for (int i = threadIdx.x; i < 2 * N1; i += kFftThreads) {
        const int col = i >= N1 ? 1 : 0, t1 = i - col * N1;
        wt[col][t1] = cconj(twiddle(((int64_t)t1 * (col ? fb : fa)) & (N - 1), N));
    }
    __syncthreads();
    float2 *S = lds_fft1(bufA, bufB, tw, N1, p.log1, lS, false);
    float2 *Z = kFftInPlace ? S : (S == bufA ? bufB : bufA);
    if (p.part != nullptr) {
        // one item per (f1, column, group slot): the sum over the group's
        // channels in this tile (a self-paired column once)
        const int c_lo = (tile << logP) * 2;
        const int c_end = min(c_lo + (2 << logP), 2 * p.np);
        const int g0 = c_lo / p.group_size;
        const int n_items = N1 * 2 * p.n_slots;
        for (int it = threadIdx.x; it < n_items; it += kFftThreads) {
            // slot fastest: a wave's lanes read different pairs and store
            // consecutive values of part
            const int slot = it % p.n_slots;
            const int col = (it / p.n_slots) & 1;
            const int f1 = it / (2 * p.n_slots);
            const int g = g0 + slot;
            const int lo = max(c_lo, g * p.group_size), hi = min(c_end, (g + 1) * p.group_size);
            if ((self && col) || lo >= hi) continue;
            const int f2 = col ? fb : fa;
            const int f1m = (N1 - f1 - (f2 > 0 ? 1 : 0)) & (N1 - 1);
            // the group's channels from a start rotated by f1 (see the
            // single-column kernel: the lanes' rows would share a bank)
            const int nch = hi - lo;
            int kk = f1 % nch;
            float2 acc = make_float2(0.0f, 0.0f);
            for (int k = 0; k < nch; ++k) {
                const int ch = lo + kk;
                kk = kk + 1 == nch ? 0 : kk + 1;
                const int pp = (ch - c_lo) >> 1;
                const int ix = (f1 << lS) | (col << logP) | pp;
                const int im = (f1m << lS) | ((col ^ 1) << logP) | pp;
                const float sg = (ch & 1) ? -1.0f : 1.0f;
                const float2 ax = S[ix], mx = cconj(S[im]), az = S[ix + sdz], mz = cconj(S[im + sdz]);
                const float2 u = make_float2(az.x + sg * mz.x, az.y + sg * mz.y);
                const float2 w = make_float2(ax.x + sg * mx.x, ax.y + sg * mx.y);
                const float2 pr = cmul(u, cconj(w));
                acc.x += pr.x;
                acc.y += pr.y;
            }
            p.part[((((int64_t)b * p.n_tiles + tile) * M + f2) * N1 + f1) * p.n_slots + slot] =
                make_float2(0.25f * acc.x, 0.25f * acc.y);
        }
    }
    // 2P divides the thread count: a thread keeps one column and pair
    const int my_col = (threadIdx.x >> logP) & 1, my_pp = threadIdx.x & pmask;
    const int my_f2 = my_col ? fb : fa;
    const int my_j = (tile << logP) + my_pp;
    const int jc = min(my_j, p.np - 1);
    const float2 *hrow0 = p.hs + (size_t)my_f2 * N1 * p.Gp + (2 * jc) / p.group_size;
    const float2 *hrow1 = p.hs + (size_t)my_f2 * N1 * p.Gp + (2 * jc + 1) / p.group_size;
    const int NP2 = N1 << lP2;
    // (in place) this thread's products, value u at i = tid + u kFftThreads,
    // written over the spectra after a barrier: they read partner values
    constexpr int UZ = kFftIpVals / 2;  // NP2 = NS / 2 <= UZ kFftThreads
    float2 zxr[kFftInPlace ? UZ : 1], zdr[kFftInPlace ? UZ : 1];
#pragma unroll
    for (int ub = 0; ub < UZ; ub += kBatch) {
        const int base = ub * kFftThreads;
        if (base >= NP2) break;
        float2 h0[kBatch], h1[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int f1 = min(base + u * kFftThreads + (int)threadIdx.x, NP2 - 1) >> lP2;
            h0[u] = hrow0[(size_t)f1 * p.Gp];
            h1[u] = hrow1[(size_t)f1 * p.Gp];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = base + u * kFftThreads + (int)threadIdx.x;
            if (i >= NP2) continue;
            const int f1 = i >> lP2;
            const int f1m = (N1 - f1 - (my_f2 > 0 ? 1 : 0)) & (N1 - 1);
            const int ix = (f1 << lS) | (my_col << logP) | my_pp;
            const int im = (f1m << lS) | ((my_col ^ 1) << logP) | my_pp;
            const float2 sm = make_float2(0.5f * (h0[u].x + h1[u].x), 0.5f * (h0[u].y + h1[u].y));
            const float2 df = make_float2(0.5f * (h0[u].x - h1[u].x), 0.5f * (h0[u].y - h1[u].y));
            const float2 ax = S[ix], mx = cconj(S[im]), az = S[ix + sdz], mz = cconj(S[im + sdz]);
            const float2 zx0 = cmul(sm, ax), zx1 = cmul(df, mx);
            const float2 zd0 = cmul(cconj(sm), az), zd1 = cmul(cconj(df), mz);
            const bool ok = my_j < p.np;
            const float2 zx = ok ? make_float2(zx0.x + zx1.x, zx0.y + zx1.y) : make_float2(0.0f, 0.0f);
            const float2 zd = ok ? make_float2(zd0.x + zd1.x, zd0.y + zd1.y) : make_float2(0.0f, 0.0f);
            if constexpr (kFftInPlace) {
                zxr[ub + u] = zx;
                zdr[ub + u] = zd;
            } else {
                Z[ix] = zx;
                Z[ix + sdz] = zd;
            }
        }
    }
    __syncthreads();
    if constexpr (kFftInPlace) {
#pragma unroll
        for (int u = 0; u < UZ; ++u) {
            const int i = threadIdx.x + u * kFftThreads;
            if (i >= NP2) continue;
            const int ix = ((i >> lP2) << lS) | (my_col << logP) | my_pp;
            Z[ix] = zxr[u];
            Z[ix + sdz] = zdr[u];
        }
        __syncthreads();
    }
    const float2 *U = lds_fft1(Z, S, tw, N1, p.log1, lS, true);
    for (int i = threadIdx.x; i < NS; i += kFftThreads) {
        const int t1 = i >> lS, col = (i >> logP) & 1, src = (i >> lP2) & 1;
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np || (self && col)) continue;
        p.ws[wpos(src, col, t1, j)] = cmul(U[i], wt[col][t1]);
    }
}

// Backward column kernel, single-column form, for even group sizes (both
// channels of every pair share a filter: H0 = H1 = H).  Per (batch, column
// f2, pair tile): the N1-point transforms of the x and dz columns, then
//     Z = H P_x[f],   DX = conj(H) P_dz[f],
// both transformed back, twiddled and stored in place; and with `part` set
// the partial sums P_dz[f] conj(P_x[f]) over the group's pairs in this tile.
// For a pair (c0, c1) of one group the real part of the inverse transform of
// P_dz conj(P_x) is the sum of the two channels' correlations (the cross
// terms are imaginary); the filter-gradient column kernel keeps only the
// Hermitian part of each group's spectrum, which is that real part.
// LDS (dynamic): one buffer (in place) of 2 N1 P values -- element (t1, src, pair) at
// (2 t1 + src) P + pair -- the N1 inner twiddles and the N1 inter-step
// twiddles W_N^(-t1 f2).
// LR > 0: the register-fed form for full tiles (2 N1 P = 4096 values, the 2P
// sequences interleaved as above) whose last stage has radix 2^LR: a thread
// keeps one source and pair, so its products need no other thread's values;
// the forward's results go to LDS only for the partial sums.
template <int LR>
__global__ __launch_bounds__(kFftThreads) void fft_bwd_col1_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int M = p.N2 * p.N3;  // columns
    const int f2 = (item / p.n_tiles) % M;
    const int b = item / (p.n_tiles * M);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1;
    const int lS = logP + 1;
    const int NS = N1 << lS;
    const int sdz = 1 << logP;
    const int64_t N = (int64_t)N1 * M;
    const int64_t area = (int64_t)p.nb * N * p.np;
    // work-area row of (f2, t1 = 0): column position as in the paired form
    const int64_t col0 = ((int64_t)b * M + (int64_t)(f2 & (p.N3 - 1)) * p.N2 + (f2 >> p.log3)) * N1;
    float2 *bufA = lds, *bufB = lds + NS, *tw = lds + kRowBufs * NS, *wt = tw + N1;
    // P divides the thread count: a thread keeps one pair (and filter row);
    // its spectrum values (value u: (f1, pair) index i = tid + u kFftThreads
    // < N1 P) are loaded before the transform
    const int my_pp = threadIdx.x & pmask;
    const int my_j = (tile << logP) + my_pp;
    const int jc = min(my_j, p.np - 1);
    const float2 *hrow = p.hs + (size_t)f2 * N1 * p.Gp + (2 * jc) / p.group_size;
    const int NP = N1 << logP;
    // the filter-gradient partial sums of this tile from the transformed
    // columns S (x at (f1 << lS) + pair, dz sdz further)
    auto partial_sums = [&](const float2 *S) {
        // one item per (f1, group slot): pairs lie inside one group
        const int c_lo = (tile << logP) * 2;
        const int c_end = min(c_lo + (2 << logP), 2 * p.np);
        const int g0 = c_lo / p.group_size;
        const int n_items = N1 * p.n_slots;
        for (int it = threadIdx.x; it < n_items; it += kFftThreads) {
            // f1 fastest: a wave's stores are consecutive values of part
            // (slot-major layout), and its lanes read at rotated pairs
            const int f1 = it % N1;
            const int slot = it / N1;
            const int g = g0 + slot;
            const int lo = max(c_lo, g * p.group_size), hi = min(c_end, (g + 1) * p.group_size);
            if (lo >= hi) continue;
            // the group's pairs, from a start rotated by f1: the lanes of a
            // wave hold different f1 (rows of the tile 8 << lS bytes apart,
            // one bank), and would otherwise read one pair at a time
            const int p0 = (lo - c_lo) >> 1, npg = ((hi - c_lo) >> 1) - p0;
            int kk = f1 % npg;
            float2 acc = make_float2(0.0f, 0.0f);
            for (int k = 0; k < npg; ++k) {
                const int ix = (f1 << lS) | (p0 + kk);
                kk = kk + 1 == npg ? 0 : kk + 1;
                const float2 pr = cmul(S[ix + sdz], cconj(S[ix]));
                acc.x += pr.x;
                acc.y += pr.y;
            }
            p.part[((((int64_t)b * p.n_tiles + tile) * p.n_slots + slot) * M + f2) * N1 + f1] = acc;
        }
    };
    if constexpr (LR > 0) {
        if (!fft_reg_ok(p.log1, lS) || fft_last_log(p.log1) != LR) return;  // the host's choice
        constexpr int lr = LR;
        const int src = (threadIdx.x >> logP) & 1;
        const bool ok = my_j < p.np;
        const int64_t base = src * area + col0 * p.np + (ok ? my_j : 0);
        float2 hr[kFftRegVals], v[kFftRegVals];
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e) hr[e] = hrow[(size_t)fft_reg_out(e, lr, p.log1, lS) * p.Gp];
#pragma unroll
        for (int u = 0; u < kFftRegVals; ++u) {
            const float2 x = p.ws[base + (int64_t)((threadIdx.x + u * kFftThreads) >> lS) * p.np];
            v[u] = ok ? x : make_float2(0.0f, 0.0f);
        }
        fill_twiddles(tw, N1);
        for (int t1 = threadIdx.x; t1 < N1; t1 += kFftThreads)
            wt[t1] = cconj(twiddle(((int64_t)t1 * f2) & (N - 1), N));
        fft_reg_first<false>(bufA, lS, v);
        __syncthreads();
        fft_reg_last<1 << LR, false>(bufA, tw, lS, 16, v);
        if (p.part != nullptr) {
            __syncthreads();  // every thread's last-stage reads are done
#pragma unroll
            for (int e = 0; e < kFftRegVals; ++e)
                bufA[(fft_reg_out(e, lr, p.log1, lS) << lS) + (threadIdx.x & ((2 << logP) - 1))] = v[e];
            __syncthreads();
            partial_sums(bufA);
        }
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e)
            v[e] = ok ? cmul(src ? cconj(hr[e]) : hr[e], v[e]) : make_float2(0.0f, 0.0f);
        fft_reg_perm<1 << LR>(v);
        __syncthreads();  // the last-stage (or partial-sum) reads are done
        fft_reg_first<true>(bufA, lS, v);
        __syncthreads();
        fft_reg_last<1 << LR, true>(bufA, tw, lS, 16, v);
        if (ok) {
            const int64_t obase = src * area + col0 * p.np + my_j;
#pragma unroll
            for (int e = 0; e < kFftRegVals; ++e) {
                const int t1 = fft_reg_out(e, lr, p.log1, lS);
                p.ws[obase + (int64_t)t1 * p.np] = cmul(v[e], wt[t1]);
            }
        }
        return;
    }
    float2 hh[kFftIpVals / 2];
#pragma unroll
    for (int u = 0; u < kFftIpVals / 2; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        if (i < NP) hh[u] = hrow[(size_t)(i >> logP) * p.Gp];
    }
    stage_in(bufA, NS, [&](int i) {
        const int src = (i >> logP) & 1;
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[src * area + (col0 + (i >> lS)) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N1);
    for (int t1 = threadIdx.x; t1 < N1; t1 += kFftThreads)
        wt[t1] = cconj(twiddle(((int64_t)t1 * f2) & (N - 1), N));
    __syncthreads();
    float2 *S = lds_fft1(bufA, bufB, tw, N1, p.log1, lS, false);
    // products to the other buffer, or (in place) over S once the partial
    // sums, which read other threads' values, are done
    float2 *Z = kFftInPlace ? S : (S == bufA ? bufB : bufA);
    if (p.part != nullptr) partial_sums(S);
    if constexpr (kFftInPlace) __syncthreads();
#pragma unroll
    for (int u = 0; u < kFftIpVals / 2; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        if (i >= NP) continue;
        const int ix = ((i >> logP) << lS) | my_pp;
        const bool ok = my_j < p.np;
        Z[ix] = ok ? cmul(hh[u], S[ix]) : make_float2(0.0f, 0.0f);
        Z[ix + sdz] = ok ? cmul(cconj(hh[u]), S[ix + sdz]) : make_float2(0.0f, 0.0f);
    }
    __syncthreads();
    const float2 *U = lds_fft1(Z, S, tw, N1, p.log1, lS, true);
    for (int i = threadIdx.x; i < NS; i += kFftThreads) {
        const int src = (i >> logP) & 1;
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        const int t1 = i >> lS;
        p.ws[src * area + (col0 + t1) * p.np + j] = cmul(U[i], wt[t1]);
    }
}

// Filter-gradient column kernel.  Per (column pair {f2, M - f2}, tile of P
// group pairs): the spectrum of each group g, S_g = the partial sums over
// the batch rows and the column tiles holding g's channels; its Hermitian
// part, whose inverse transform is the real part of S_g's
// (H_g[f] = (S_g[f] + conj(S_g[-f]))/2); two groups packed as one complex
// sequence, Q = H_2m + i H_2m+1 (real and imaginary parts of the result
// are then the two gradients); the inverse N1-point transform along f1 and
// the twiddle W_N^(-t1 f2), stored as a one-row work area of Gp/2 pairs.
// p.np = Gp/2 here; pb_log, pb_tiles and n_slots describe the backward
// column tiles that wrote `part`.
// LDS (dynamic): the sums (N1 (4P + 1) values), two buffers of 2 N1 P
// values, the N1 inner twiddles and 2 N1 inter-step twiddles.
__global__ __launch_bounds__(kFftThreads) void fft_dh_cols_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int M = p.N2 * p.N3;
    const int c = item / p.n_tiles;
    const int logP = p.logP, N1 = p.N1;
    const int lG = logP + 1;            // groups of the tile (log2)
    const int lS = logP + 2;            // (col, group) sequences of the sums
    const int lQ = logP + 1;            // (col, group pair) sequences of the transform
    const int64_t N = (int64_t)N1 * M;
    const int fa = c, fb = (M - c) & (M - 1);
    const bool self = fa == fb;
    auto cpos = [&](int f) -> int64_t { return (int64_t)(f & (p.N3 - 1)) * p.N2 + (f >> p.log3); };
    // sums of (f1, col, group) at f1 SP + (col << lG) + group: rows padded
    // by one value, so the f1-fastest writes below spread over the banks
    const int SP = (2 << lG) + 1;
    auto sidx = [&](int f1, int col, int g) -> int { return f1 * SP + (col << lG) + g; };
    float2 *sums = lds, *bufA = lds + N1 * SP, *bufB = bufA + (N1 << lQ), *tw = bufB + (N1 << lQ);
    float2 *wt[2] = {tw + N1, tw + 2 * N1};
    const int cpt = 2 << p.pb_log;      // channels per backward column tile
    for (int e = threadIdx.x; e < (N1 << lS); e += kFftThreads) {
        // f1 fastest: a wave reads consecutive partials (slot-major layout)
        // or partials n_slots apart, whose lines the workgroup's other
        // groups read as well
        const int f1 = e % N1, r = e / N1;
        const int col = r >> lG, gl = r & ((1 << lG) - 1);
        const int g = (tile << lG) + gl;
        float2 acc = make_float2(0.0f, 0.0f);
        if (g < p.G) {
            const int f2 = (self || !col) ? fa : fb;
            const int t_lo = (g * p.group_size) / cpt, t_hi = ((g + 1) * p.group_size - 1) / cpt;
            for (int b = 0; b < p.nb; ++b) {
                for (int t = t_lo; t <= t_hi; ++t) {
                    const int slot = g - (t * cpt) / p.group_size;
                    const int64_t bt = (int64_t)b * p.pb_tiles + t;
                    const float2 v = p.part_slot_major ? p.part[((bt * p.n_slots + slot) * M + f2) * N1 + f1]
                                                       : p.part[((bt * M + f2) * N1 + f1) * p.n_slots + slot];
                    acc.x += v.x;
                    acc.y += v.y;
                }
            }
        }
        sums[sidx(f1, col, gl)] = acc;
    }
    fill_twiddles(tw, N1);
    for (int i = threadIdx.x; i < 2 * N1; i += kFftThreads) {
        const int col = i >= N1 ? 1 : 0, t1 = i - col * N1;
        wt[col][t1] = cconj(twiddle(((int64_t)t1 * (col ? fb : fa)) & (N - 1), N));
    }
    __syncthreads();
    const int gmask = (1 << logP) - 1;
    for (int e = threadIdx.x; e < (N1 << lQ); e += kFftThreads) {
        const int f1 = e >> lQ, col = (e >> logP) & 1, m = e & gmask;
        const int f2 = col ? fb : fa;
        const int f1m = (N1 - f1 - (f2 > 0 ? 1 : 0)) & (N1 - 1);
        const int ia = sidx(f1, col, 2 * m);
        const int ib = sidx(f1m, col ^ 1, 2 * m);
        const float2 s0 = sums[ia], s1 = sums[ia + 1], r0 = sums[ib], r1 = sums[ib + 1];
        // H = (S[f] + conj(S[-f]))/2 for both groups, then H0 + i H1
        const float2 h0 = make_float2(0.5f * (s0.x + r0.x), 0.5f * (s0.y - r0.y));
        const float2 h1 = make_float2(0.5f * (s1.x + r1.x), 0.5f * (s1.y - r1.y));
        bufA[e] = make_float2(h0.x - h1.y, h0.y + h1.x);
    }
    __syncthreads();
    const float2 *U = lds_fft(bufA, bufB, tw, N1, p.log1, lQ, true);
    for (int e = threadIdx.x; e < (N1 << lQ); e += kFftThreads) {
        const int t1 = e >> lQ, col = (e >> logP) & 1;
        const int j = (tile << logP) + (e & gmask);
        if (j >= p.np || (self && col)) continue;
        p.ws[(cpos(col ? fb : fa) * N1 + t1) * p.np + j] = cmul(U[e], wt[col][t1]);
    }
}

// The filter gradient from the last inverse pass's [taps][Gp] layout to
// [G][l_h], zero for taps t >= taps (l_h > L: no row reaches them).  64 x 64
// tiles through LDS: reads run along filters, writes along taps.
__global__ __launch_bounds__(256) void fft_dh_transpose_kernel(const float *dhT, float *dh, int G, int Gp, int l_h,
                                                              int taps, int n_tblk) {
    __shared__ float tile[64][65];
    const int t0 = (int)(blockIdx.x % n_tblk) * 64, g0 = (int)(blockIdx.x / n_tblk) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    // all 16 loads of a thread in flight together
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int t = t0 + ty + 4 * u, g = g0 + tx;
        v[u] = (t < taps && g < Gp) ? dhT[(size_t)t * Gp + g] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) tile[ty + 4 * u][tx] = v[u];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int g = g0 + ty + 4 * u, t = t0 + tx;
        if (g < G && t < l_h) dh[(size_t)g * l_h + t] = tile[tx][ty + 4 * u];
    }
}

// Filter-gradient taps from `from` on: zero (a call with no rows).
__global__ __launch_bounds__(256) void fft_dh_tail_kernel(float *dh, int64_t G, int64_t l_h, int64_t from) {
    const int64_t w = l_h - from;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < G * w) dh[(i / w) * l_h + from + i % w] = 0.0f;
}

// Output of the last inverse pass for channel pair j at row t (values
// already scaled).  MODE 0: y = q z (the forward; the backward's dq with dy in
// q's place).  MODE 1: the backward's dk = z v and dv = z k (z = dx).  MODE 2:
// the filter gradient transposed, fp32 [taps][Gp], groups 2j and 2j + 1 at
// tap t (consecutive lanes write consecutive group pairs of one tap;
// fft_dh_transpose_kernel then writes [G][l_h]).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}
// The gates of one output (raw bits: a bf16 pair in .x, or an fp32 pair),
// loaded before the last transform so that their latency is hidden behind it.
template <bool F32, int MODE> struct Gates {
    static constexpr int NG = MODE == 2 ? 0 : (MODE == 1 ? 2 : 1);   // gates per output
    static constexpr int NW = NG * (F32 ? 2 : 1);                    // 4-byte words
    uint32_t w[NW > 0 ? NW : 1];
};
template <bool F32, int MODE>
__device__ inline void load_gates(const FftParams &p, int b, int64_t t, int j, Gates<F32, MODE> &r) {
    if constexpr (MODE != 2) {
        const size_t o = ((size_t)b * (size_t)p.L + (size_t)t) * (size_t)p.D + 2 * (size_t)j;
        const void *ga = MODE == 0 ? p.q : p.v;
        if constexpr (F32) {
            const uint2 a = *(const uint2 *)((const float *)ga + o);
            r.w[0] = a.x;
            r.w[1] = a.y;
            if constexpr (MODE == 1) {
                const uint2 c = *(const uint2 *)((const float *)p.k + o);
                r.w[2] = c.x;
                r.w[3] = c.y;
            }
        } else {
            r.w[0] = *(const uint32_t *)((const uint16_t *)ga + o);
            if constexpr (MODE == 1) r.w[1] = *(const uint32_t *)((const uint16_t *)p.k + o);
        }
    }
}
template <bool F32, int MODE>
__device__ inline void store_out(const FftParams &p, int b, int64_t t, int j, float z0, float z1,
                                 const Gates<F32, MODE> &g) {
    if constexpr (MODE == 2) {
        *(float2 *)((float *)p.y + (size_t)t * (size_t)p.Gp + 2 * (size_t)j) = make_float2(z0, z1);
        return;
    }
    const size_t o = ((size_t)b * (size_t)p.L + (size_t)t) * (size_t)p.D + 2 * (size_t)j;
    if constexpr (F32) {
        *(float2 *)((float *)p.y + o) = make_float2(__uint_as_float(g.w[0]) * z0, __uint_as_float(g.w[1]) * z1);
        if constexpr (MODE == 1)
            *(float2 *)((float *)p.y2 + o) = make_float2(__uint_as_float(g.w[2]) * z0, __uint_as_float(g.w[3]) * z1);
    } else {
        *(uint32_t *)((uint16_t *)p.y + o) =
            pack_bf16x2(__uint_as_float(g.w[0] << 16) * z0, __uint_as_float(g.w[0] & 0xffff0000u) * z1);
        if constexpr (MODE == 1)
            *(uint32_t *)((uint16_t *)p.y2 + o) =
                pack_bf16x2(__uint_as_float(g.w[1] << 16) * z0, __uint_as_float(g.w[1] & 0xffff0000u) * z1);
    }
}

// Three-level split (large N): N = N1 N2 N3, t = t1 + N1 t2 + N1 N2 t3.
// The M = N2 N3 point transform along t2 + N2 t3 that the row kernel does
// in one piece is done in two passes, as a four-step of its own:
//   rows3 (per t1, t2):  N3-point FFT over t3, twiddle W_M^(t2 f3), store at
//                        work-area position f3 N2 + t2;
//   mid   (per t1, f3):  N2-point FFT over t2, twiddle W_N^(t1 c) with column
//                        c = f3 + N3 f2, store at position f3 N2 + f2;
// after which column c (position (c mod N3) N2 + c / N3) is what the column
// kernel expects.  The inverse runs mid (inverse, twiddle conj W_M^(t2 f3))
// and out3 (inverse N3-point FFT over f3, scale, gate, store).
// LDS (dynamic) of either: one buffer (in place) of N3 P (N2 P) values, the inner
// twiddles and the N3 (N2) inter-step twiddles.
template <bool F32, int SRC, bool REG>
__global__ __launch_bounds__(kFftThreads) void fft_rows3_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int t2 = (item / p.n_tiles) % p.N2;
    const int t1 = (item / (p.n_tiles * p.N2)) % p.N1;
    const int b = item / (p.n_tiles * p.N2 * p.N1);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1, N2 = p.N2, N3 = p.N3;
    const int NP = N3 << logP;
    const int64_t M = (int64_t)N2 * N3;
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + kRowBufs * NP, *wt = tw + N3;
    if constexpr (REG) {
        // full tile: loads into the first stage, the last stage into the stores
        if (!fft_reg_ok(p.log3, logP)) return;  // the host launches this form only for full tiles
        const int j = (tile << logP) + (threadIdx.x & pmask);
        float2 v[kFftRegVals];
#pragma unroll
        for (int u = 0; u < kFftRegVals; ++u)
            v[u] = load_pair<F32, SRC>(
                p, b, t1 + (int64_t)N1 * (t2 + (int64_t)N2 * ((threadIdx.x + u * kFftThreads) >> logP)), j);
        fill_twiddles(tw, N3);
        for (int f3 = threadIdx.x; f3 < N3; f3 += kFftThreads) wt[f3] = twiddle(((int64_t)t2 * f3) & (M - 1), M);
        fft_reg_first<false>(buf0, logP, v);
        __syncthreads();
        fft_reg_rest<false>(buf0, tw, p.log3, logP, v);
        if (j < p.np) {
            const int lr = fft_last_log(p.log3);
#pragma unroll
            for (int e = 0; e < kFftRegVals; ++e) {
                const int f3 = fft_reg_out(e, lr, p.log3, logP);
                p.ws[(((int64_t)b * M + (int64_t)f3 * N2 + t2) * N1 + t1) * p.np + j] = cmul(v[e], wt[f3]);
            }
        }
        return;
    }
    stage_in(buf0, NP, [&](int i) {
        return load_pair<F32, SRC>(p, b, t1 + (int64_t)N1 * (t2 + (int64_t)N2 * (i >> logP)),
                                   (tile << logP) + (i & pmask));
    });
    fill_twiddles(tw, N3);
    for (int f3 = threadIdx.x; f3 < N3; f3 += kFftThreads) wt[f3] = twiddle(((int64_t)t2 * f3) & (M - 1), M);
    __syncthreads();
    const float2 *X = lds_fft1(buf0, buf1, tw, N3, p.log3, logP, false);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int f3 = i >> logP;
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        p.ws[(((int64_t)b * M + (int64_t)f3 * N2 + t2) * N1 + t1) * p.np + j] = cmul(X[i], wt[f3]);
    }
}

template <bool INV, bool REG>
__global__ __launch_bounds__(kFftThreads) void fft_mid_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int f3 = (item / p.n_tiles) % p.N3;
    const int t1 = (item / (p.n_tiles * p.N3)) % p.N1;
    const int b = item / (p.n_tiles * p.N3 * p.N1);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1, N2 = p.N2, N3 = p.N3;
    const int NP = N2 << logP;
    const int64_t M = (int64_t)N2 * N3;
    const int64_t N = M * N1;
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + kRowBufs * NP, *wt = tw + N2;
    const int64_t row0 = (int64_t)b * M + (int64_t)f3 * N2;  // position of index 0 along t2 / f2
    if constexpr (REG) {
        // full tile: loads into the first stage, the last stage into the stores
        if (!fft_reg_ok(p.log2, logP)) return;  // the host launches this form only for full tiles
        const int j = (tile << logP) + (threadIdx.x & pmask);
        const bool ok = j < p.np;
        float2 v[kFftRegVals];
#pragma unroll
        for (int u = 0; u < kFftRegVals; ++u) {
            const float2 x = p.ws[((row0 + ((threadIdx.x + u * kFftThreads) >> logP)) * N1 + t1) * p.np + (ok ? j : 0)];
            v[u] = ok ? x : make_float2(0.0f, 0.0f);
        }
        fill_twiddles(tw, N2);
        for (int u = threadIdx.x; u < N2; u += kFftThreads)
            wt[u] = INV ? cconj(twiddle(((int64_t)u * f3) & (M - 1), M))
                        : twiddle(((int64_t)t1 * (f3 + (int64_t)N3 * u)) & (N - 1), N);
        fft_reg_first<INV>(buf0, logP, v);
        __syncthreads();
        fft_reg_rest<INV>(buf0, tw, p.log2, logP, v);
        if (ok) {
            const int lr = fft_last_log(p.log2);
#pragma unroll
            for (int e = 0; e < kFftRegVals; ++e) {
                const int u = fft_reg_out(e, lr, p.log2, logP);
                p.ws[((row0 + u) * N1 + t1) * p.np + j] = cmul(v[e], wt[u]);
            }
        }
        return;
    }
    stage_in(buf0, NP, [&](int i) {
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[((row0 + (i >> logP)) * N1 + t1) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N2);
    for (int u = threadIdx.x; u < N2; u += kFftThreads)
        wt[u] = INV ? cconj(twiddle(((int64_t)u * f3) & (M - 1), M))
                    : twiddle(((int64_t)t1 * (f3 + (int64_t)N3 * u)) & (N - 1), N);
    __syncthreads();
    const float2 *X = lds_fft1(buf0, buf1, tw, N2, p.log2, logP, INV);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int u = i >> logP;
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        p.ws[((row0 + u) * N1 + t1) * p.np + j] = cmul(X[i], wt[u]);
    }
}

template <bool F32, int MODE, bool REG>
__global__ __launch_bounds__(kFftThreads) void fft_out3_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int t2 = (item / p.n_tiles) % p.N2;
    const int t1 = (item / (p.n_tiles * p.N2)) % p.N1;
    const int b = item / (p.n_tiles * p.N2 * p.N1);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1, N2 = p.N2, N3 = p.N3;
    const int NP = N3 << logP;
    const int64_t M = (int64_t)N2 * N3;
    const float scale = 1.0f / ((float)N1 * (float)M);
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + kRowBufs * NP;
    if constexpr (REG) {
        // full tile: loads into the first stage, the last stage into the stores
        if (!fft_reg_ok(p.log3, logP)) return;  // the host launches this form only for full tiles
        const int jj = (tile << logP) + (threadIdx.x & pmask);
        const bool ok = jj < p.np;
        const int lr = fft_last_log(p.log3);
        auto row_of = [&](int e) -> int64_t {
            return t1 + (int64_t)N1 * (t2 + (int64_t)N2 * fft_reg_out(e, lr, p.log3, logP));
        };
        Gates<F32, MODE> gr[kFftRegVals];
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e)
            if (ok && row_of(e) < p.L) load_gates<F32, MODE>(p, b, row_of(e), jj, gr[e]);
        float2 v[kFftRegVals];
#pragma unroll
        for (int u = 0; u < kFftRegVals; ++u) {
            const int f3 = (threadIdx.x + u * kFftThreads) >> logP;
            const float2 x = p.ws[(((int64_t)b * M + (int64_t)f3 * N2 + t2) * N1 + t1) * p.np + (ok ? jj : 0)];
            v[u] = ok ? x : make_float2(0.0f, 0.0f);
        }
        fill_twiddles(tw, N3);
        fft_reg_first<true>(buf0, logP, v);
        __syncthreads();
        fft_reg_rest<true>(buf0, tw, p.log3, logP, v);
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e)
            if (ok && row_of(e) < p.L)
                store_out<F32, MODE>(p, b, row_of(e), jj, v[e].x * scale, v[e].y * scale, gr[e]);
        return;
    }
    // output u of this thread: i = tid + u kFftThreads (NP <= kFftIpVals kFftThreads)
    auto out_row = [&](int i) -> int64_t { return t1 + (int64_t)N1 * (t2 + (int64_t)N2 * (i >> logP)); };
    Gates<F32, MODE> gv[kFftIpVals];
#pragma unroll
    for (int u = 0; u < kFftIpVals; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        const int j = (tile << logP) + (i & pmask);
        if (i < NP && j < p.np && out_row(i) < p.L) load_gates<F32, MODE>(p, b, out_row(i), j, gv[u]);
    }
    stage_in(buf0, NP, [&](int i) {
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[(((int64_t)b * M + (int64_t)(i >> logP) * N2 + t2) * N1 + t1) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N3);
    __syncthreads();
    const float2 *z = lds_fft1(buf0, buf1, tw, N3, p.log3, logP, true);
#pragma unroll
    for (int u = 0; u < kFftIpVals; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        const int j = (tile << logP) + (i & pmask);
        if (i < NP && j < p.np && out_row(i) < p.L)
            store_out<F32, MODE>(p, b, out_row(i), j, z[i].x * scale, z[i].y * scale, gv[u]);
    }
}

// Kernel 3: inverse transform along f2 for one t1, scale, gate, store.
// LDS (dynamic): one buffer (in place) of N2 P values and the N2 inner twiddles.
template <bool F32, int MODE, bool REG>
__global__ __launch_bounds__(kFftThreads) void fft_out_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int t1 = (item / p.n_tiles) % p.N1;
    const int b = item / (p.n_tiles * p.N1);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1, N2 = p.N2;
    const int NP = N2 << logP;
    const float scale = 1.0f / ((float)N1 * (float)N2);
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + kRowBufs * NP;
    if constexpr (REG) {
        // full tile: loads into the first stage, the last stage into the stores
        if (!fft_reg_ok(p.log2, logP)) return;  // the host launches this form only for full tiles
        const int jj = (tile << logP) + (threadIdx.x & pmask);
        const bool ok = jj < p.np;
        const int lr = fft_last_log(p.log2);
        Gates<F32, MODE> gr[kFftRegVals];
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e) {
            const int64_t t = t1 + (int64_t)N1 * fft_reg_out(e, lr, p.log2, logP);
            if (ok && t < p.L) load_gates<F32, MODE>(p, b, t, jj, gr[e]);
        }
        float2 v[kFftRegVals];
#pragma unroll
        for (int u = 0; u < kFftRegVals; ++u) {
            const float2 x =
                p.ws[(((int64_t)b * N2 + ((threadIdx.x + u * kFftThreads) >> logP)) * N1 + t1) * p.np + (ok ? jj : 0)];
            v[u] = ok ? x : make_float2(0.0f, 0.0f);
        }
        fill_twiddles(tw, N2);
        fft_reg_first<true>(buf0, logP, v);
        __syncthreads();
        fft_reg_rest<true>(buf0, tw, p.log2, logP, v);
#pragma unroll
        for (int e = 0; e < kFftRegVals; ++e) {
            const int64_t t = t1 + (int64_t)N1 * fft_reg_out(e, lr, p.log2, logP);
            if (ok && t < p.L) store_out<F32, MODE>(p, b, t, jj, v[e].x * scale, v[e].y * scale, gr[e]);
        }
        return;
    }
    // output u of this thread: i = tid + u kFftThreads (NP <= kFftIpVals kFftThreads)
    Gates<F32, MODE> gv[kFftIpVals];
#pragma unroll
    for (int u = 0; u < kFftIpVals; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        const int j = (tile << logP) + (i & pmask);
        const int64_t t = t1 + (int64_t)N1 * (i >> logP);
        if (i < NP && j < p.np && t < p.L) load_gates<F32, MODE>(p, b, t, j, gv[u]);
    }
    stage_in(buf0, NP, [&](int i) {
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[(((int64_t)b * N2 + (i >> logP)) * N1 + t1) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N2);
    __syncthreads();
    const float2 *z = lds_fft1(buf0, buf1, tw, N2, p.log2, logP, true);
#pragma unroll
    for (int u = 0; u < kFftIpVals; ++u) {
        const int i = threadIdx.x + u * kFftThreads;
        const int j = (tile << logP) + (i & pmask);
        const int64_t t = t1 + (int64_t)N1 * (i >> logP);
        if (i < NP && j < p.np && t < p.L) store_out<F32, MODE>(p, b, t, j, z[i].x * scale, z[i].y * scale, gv[u]);
    }
}

struct FftPlan {
    int64_t N, ws_pairs, hs_bytes, ws_bytes;
    int N1, N2, N3, log1, log2, log3;
    bool three;                      // three-level split (N3 > 1)
    int P_rows, P_mid, P_cols, P_col1;          // pairs per workgroup: row (rows3/out3), middle,
    int lds_rows, lds_mid, lds_cols, lds_col1;  // column (paired, single) kernels; their LDS bytes
    bool reg_rows, reg_col1;                    // full tiles: the register-fed forms of the row and
                                                // output kernels (two-level) and of the single-column kernel,
    bool reg_rows3, reg_mid;                    // and of the three-level row / output and middle kernels
    // backward: column kernel (pairs per tile, tiles, group slots per tile),
    // filter-gradient column kernel (group pairs per tile), LDS, and the
    // workspace: spectra, two work areas, partial sums
    int P_bwd, P_dh, lds_bwd, lds_dh;
    bool bwd_col1;                   // the backward's single-column form (even group sizes)
    bool reg_bwd1;                   // ... in its register-fed form (full tiles)
    int64_t pb_tiles, n_slots, area_bytes, part_bytes, bwd_ws_bytes;
};

// Largest N done with the two-level split (columns of at most 256 points);
// above it the three-level split keeps every transform at 256 points or less.
constexpr int kFftTwoLevelMaxLogN = 16;

// Pairs per workgroup: LDS of about kFftBudget complex values (several
// workgroups per CU), at most 64 pairs, no more than the pairs there are; a
// single pair when even that exceeds the budget (the largest transforms).
int pick_pairs(int M, int buffers, int64_t pairs, int budget = kFftBudget) {
    int P = 64;
    while (P > 1 && (int64_t)buffers * M * P > budget) P >>= 1;
    while (P > 1 && P / 2 >= pairs) P >>= 1;
    return P;
}

int ilog2(int64_t n) {
    int r = 0;
    while (((int64_t)1 << r) < n) ++r;
    return r;
}

// Transform length, its split and the pair tile (shared by all passes).
int fft_plan(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, int dtype, FftPlan *pl) {
    if (dtype != HYENA_DTYPE_BF16 && dtype != HYENA_DTYPE_F32) return HYENA_ERR_DTYPE;
    if (B < 0 || L < 0 || D < 0) return HYENA_ERR_SHAPE;
    if (group_size < 1 || D % group_size != 0) return HYENA_ERR_GROUP;
    if (l_h < 1) return HYENA_ERR_FILTER_LEN;
    if (D % 2 != 0) return HYENA_ERR_UNSUPPORTED;  // channels travel in pairs
    // the kernels take the filter row pitch as a 32-bit count; the sequence
    // must fit one transform (checked before L + taps - 1 is formed)
    if (l_h > INT32_MAX || L > ((int64_t)1 << kFftMaxLogN)) return HYENA_ERR_UNSUPPORTED;
    if (B > 0 && L > 0 && D > 0) {
        const int64_t lim = INT64_MAX / 8;  // element count times 4-byte elements, with room
        if (L > lim / D || B > lim / (L * D)) return HYENA_ERR_SHAPE;
    }
    if (l_h > (INT64_MAX / 8) / (D / group_size > 0 ? D / group_size : 1)) return HYENA_ERR_SHAPE;
    const int64_t taps = l_h < L ? l_h : L;         // taps past row L - 1 never contribute
    const int logN = ilog2(L + taps - 1 > 4 ? L + taps - 1 : 4);
    if (logN > kFftMaxLogN) return HYENA_ERR_UNSUPPORTED;
    if (D > INT32_MAX / 2 || B > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
    pl->N = (int64_t)1 << logN;
    pl->three = logN > kFftTwoLevelMaxLogN;
    if (pl->three) {
        pl->log1 = (logN + 2) / 3;
        pl->log2 = (logN - pl->log1 + 1) / 2;
        pl->log3 = logN - pl->log1 - pl->log2;
    } else {
        pl->log1 = (logN + 1) / 2;
        pl->log2 = logN / 2;
        pl->log3 = 0;
    }
    pl->N1 = 1 << pl->log1;
    pl->N2 = 1 << pl->log2;
    pl->N3 = 1 << pl->log3;
    const int64_t G = D / group_size;
    const int64_t pairs = D / 2 > (G + 1) / 2 ? D / 2 : (G + 1) / 2;
    const int Mr = pl->three ? pl->N3 : pl->N2;  // transform length of the row (and output) kernels
    pl->P_rows = pick_pairs(Mr, kRowBufs, pairs);
    pl->P_mid = pick_pairs(pl->N2, kRowBufs, pairs);
    pl->P_cols = pick_pairs(pl->N1, 2 * kRowBufs, pairs, kFftColsBudget);
    pl->lds_rows = (kRowBufs * Mr * pl->P_rows + 2 * Mr) * (int)sizeof(float2);
    pl->lds_mid = (kRowBufs * pl->N2 * pl->P_mid + 2 * pl->N2) * (int)sizeof(float2);
    pl->lds_cols = (2 * kRowBufs * pl->N1 * pl->P_cols + 3 * pl->N1) * (int)sizeof(float2);
    pl->P_col1 = pick_pairs(pl->N1, kRowBufs, pairs);
    pl->lds_col1 = (kRowBufs * pl->N1 * pl->P_col1 + 2 * pl->N1) * (int)sizeof(float2);
    pl->reg_rows = !pl->three && pl->log2 >= 5 && pl->log2 <= 8 && pl->N2 * pl->P_rows == kFftRegVals * kFftThreads;
    pl->reg_col1 = pl->log1 >= 5 && pl->log1 <= 8 && pl->N1 * pl->P_col1 == kFftRegVals * kFftThreads;
    pl->reg_rows3 = pl->three && pl->log3 >= 5 && pl->log3 <= 8 && pl->N3 * pl->P_rows == kFftRegVals * kFftThreads;
    pl->reg_mid = pl->three && pl->log2 >= 5 && pl->log2 <= 8 && pl->N2 * pl->P_mid == kFftRegVals * kFftThreads;
    // the output kernels hold the gates of Mr P / kFftThreads outputs per
    // thread, the single-column kernel N1 P / kFftThreads filter-spectrum values
    if ((int64_t)Mr * pl->P_rows > kFftIpVals * kFftThreads ||
        (int64_t)pl->N1 * pl->P_col1 > kFftIpVals * kFftThreads ||
        (int64_t)2 * pl->N1 * pl->P_cols > kFftIpVals * kFftThreads)
        return HYENA_ERR_UNSUPPORTED;
    // an in-place stage holds M P / kFftThreads values per thread
    if (kFftInPlace && ((int64_t)Mr * pl->P_rows > kFftIpVals * kFftThreads ||
                        (int64_t)pl->N2 * pl->P_mid > kFftIpVals * kFftThreads ||
                        (int64_t)pl->N1 * pl->P_col1 > kFftIpVals * kFftThreads))
        return HYENA_ERR_UNSUPPORTED;
    if (pl->lds_rows > kFftMaxLdsBytes || pl->lds_cols > kFftMaxLdsBytes || pl->lds_mid > kFftMaxLdsBytes ||
        pl->lds_col1 > kFftMaxLdsBytes)
        return HYENA_ERR_UNSUPPORTED;
    const int64_t Gp = G + (G & 1);
    pl->ws_pairs = B * (D / 2) > Gp / 2 ? B * (D / 2) : Gp / 2;
    // N (ws_pairs + Gp) complex values of 8 bytes must not overflow
    if (pl->ws_pairs > (INT64_MAX / 16) / pl->N - Gp) return HYENA_ERR_SHAPE;
    pl->hs_bytes = pl->N * Gp * (int64_t)sizeof(float2);
    pl->ws_bytes = pl->N * pl->ws_pairs * (int64_t)sizeof(float2) + pl->hs_bytes;
    return HYENA_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// The backward's additions to the plan (after fft_plan succeeded).
int fft_bwd_plan(int64_t B, int64_t D, int64_t group_size, FftPlan *pl) {
    const int64_t G = D / group_size, Gp = G + (G & 1);
    const int64_t pairs = D / 2;
    // even group sizes: the single-column form (4 N1 P values of LDS), else the paired one (8 N1 P)
    pl->bwd_col1 = group_size % 2 == 0;
    if (pl->bwd_col1) {
        pl->P_bwd = pick_pairs(pl->N1, 2 * kRowBufs, pairs, kFftBwdBudget);
        pl->lds_bwd = (2 * kRowBufs * pl->N1 * pl->P_bwd + 2 * pl->N1) * (int)sizeof(float2);
        if ((int64_t)2 * pl->N1 * pl->P_bwd > kFftIpVals * kFftThreads) return HYENA_ERR_UNSUPPORTED;
        pl->reg_bwd1 = pl->log1 >= 5 && pl->log1 <= 8 && 2 * pl->N1 * pl->P_bwd == kFftRegVals * kFftThreads;
    } else {
        pl->reg_bwd1 = false;
        pl->P_bwd = pick_pairs(pl->N1, 4 * kRowBufs, pairs, kFftBwdBudget);
        pl->lds_bwd = (4 * kRowBufs * pl->N1 * pl->P_bwd + 3 * pl->N1) * (int)sizeof(float2);
        if ((int64_t)4 * pl->N1 * pl->P_bwd > kFftIpVals * kFftThreads) return HYENA_ERR_UNSUPPORTED;
    }
    pl->P_dh = pick_pairs(pl->N1, 8, Gp / 2, kFftColsBudget);
    pl->lds_dh = (8 * pl->N1 * pl->P_dh + 4 * pl->N1) * (int)sizeof(float2);
    if (pl->lds_bwd > kFftMaxLdsBytes || pl->lds_dh > kFftMaxLdsBytes) return HYENA_ERR_UNSUPPORTED;
    pl->pb_tiles = (pairs + pl->P_bwd - 1) / pl->P_bwd;
    // groups a tile of 2P channels can touch
    const int64_t span = (2 * (int64_t)pl->P_bwd - 1 + group_size - 1) / group_size + 1;
    pl->n_slots = span < G ? span : G;
    // B N (pairs + pb_tiles n_slots) complex values plus the spectra must not overflow
    const int64_t per_n = 2 * pairs + pl->pb_tiles * pl->n_slots;
    if (B > 0 && per_n > ((INT64_MAX / 16) / pl->N - Gp) / B) return HYENA_ERR_SHAPE;
    pl->area_bytes = B * pl->N * pairs * (int64_t)sizeof(float2);
    pl->part_bytes = B * pl->N * pl->pb_tiles * pl->n_slots * (int64_t)sizeof(float2);
    pl->bwd_ws_bytes = pl->hs_bytes + 2 * pl->area_bytes + pl->part_bytes;
    return HYENA_OK;
}

// The filters to [taps][Gp] fp32 at hT (taps Gp 4 <= 8 N Gp bytes: the
// spectra's region).
int transpose_filters(const void *h, bool f32, int64_t G, int64_t Gp, int64_t l_h, int64_t taps, void *hT,
                      hipStream_t s) {
    const int64_t gx = (taps + 63) / 64, gy = (Gp + 63) / 64;
    if (gx * gy > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(f32 ? fft_filter_transpose_kernel<true> : fft_filter_transpose_kernel<false>,
                       dim3((unsigned)(gx * gy)), dim3(256), 0, s, h, (float *)hT, (int)G, (int)Gp, (int)l_h,
                       (int)taps, (int)gx);
    return hipGetLastError() == hipSuccess ? HYENA_OK : HYENA_ERR_LAUNCH;
}

// The row, output and single-column kernels for a plan: the register-fed
// form for full tiles.
template <int SRC> const void *rows_kernel(bool f32, bool reg) {
    if (f32) return reg ? (const void *)fft_rows_kernel<true, SRC, true> : (const void *)fft_rows_kernel<true, SRC, false>;
    return reg ? (const void *)fft_rows_kernel<false, SRC, true> : (const void *)fft_rows_kernel<false, SRC, false>;
}
template <int MODE> const void *out_kernel(bool f32, bool reg) {
    if constexpr (MODE == 2) {  // the filter gradient: fp32 output
        return reg ? (const void *)fft_out_kernel<true, 2, true> : (const void *)fft_out_kernel<true, 2, false>;
    } else {
        if (f32)
            return reg ? (const void *)fft_out_kernel<true, MODE, true> : (const void *)fft_out_kernel<true, MODE, false>;
        return reg ? (const void *)fft_out_kernel<false, MODE, true> : (const void *)fft_out_kernel<false, MODE, false>;
    }
}
template <int SRC> const void *rows3_kernel(bool f32, bool reg) {
    if (f32) return reg ? (const void *)fft_rows3_kernel<true, SRC, true> : (const void *)fft_rows3_kernel<true, SRC, false>;
    return reg ? (const void *)fft_rows3_kernel<false, SRC, true> : (const void *)fft_rows3_kernel<false, SRC, false>;
}
template <int MODE> const void *out3_kernel(bool f32, bool reg) {
    if constexpr (MODE == 2) {  // the filter gradient: fp32 output
        return reg ? (const void *)fft_out3_kernel<true, 2, true> : (const void *)fft_out3_kernel<true, 2, false>;
    } else {
        if (f32)
            return reg ? (const void *)fft_out3_kernel<true, MODE, true> : (const void *)fft_out3_kernel<true, MODE, false>;
        return reg ? (const void *)fft_out3_kernel<false, MODE, true> : (const void *)fft_out3_kernel<false, MODE, false>;
    }
}
template <bool INV> const void *mid_kernel(bool reg) {
    return reg ? (const void *)fft_mid_kernel<INV, true> : (const void *)fft_mid_kernel<INV, false>;
}
const void *bwd_col1_kernel(bool reg, int log1) {
    if (!reg) return (const void *)fft_bwd_col1_kernel<0>;
    switch (fft_last_log(log1)) {
    case 1: return (const void *)fft_bwd_col1_kernel<1>;
    case 2: return (const void *)fft_bwd_col1_kernel<2>;
    case 3: return (const void *)fft_bwd_col1_kernel<3>;
    default: return (const void *)fft_bwd_col1_kernel<4>;
    }
}
const void *col1_kernel(bool reg, int log1) {
    if (!reg) return (const void *)fft_col1_kernel<0>;
    switch (fft_last_log(log1)) {
    case 1: return (const void *)fft_col1_kernel<1>;
    case 2: return (const void *)fft_col1_kernel<2>;
    case 3: return (const void *)fft_col1_kernel<3>;
    default: return (const void *)fft_col1_kernel<4>;
    }
}

// One launch: pair tile P, grid (batch rows x units x tiles), dynamic LDS.
int fft_launch(const void *fn, FftParams q_, int P, int64_t units, int64_t nb, int lds, hipStream_t s) {
    q_.logP = 0;
    while ((1 << q_.logP) < P) ++q_.logP;
    q_.n_tiles = (q_.np + P - 1) / P;
    const int64_t grid = nb * units * q_.n_tiles;
    if (grid > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
    if (lds > 64 * 1024 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return HYENA_ERR_LAUNCH;
    void *args[] = {&q_};
    if (hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kFftThreads), args, (size_t)lds, s) != hipSuccess)
        return HYENA_ERR_LAUNCH;
    return HYENA_OK;
}

}  // namespace

extern "C" {

int hyena_conv_fwd_long_workspace(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, int dtype,
                                  int64_t *bytes_out) {
    FftPlan pl;
    const int st = fft_plan(B, L, D, group_size, l_h, dtype, &pl);
    if (st != HYENA_OK) return st;
    if (bytes_out) *bytes_out = (B == 0 || L == 0 || D == 0) ? 0 : pl.ws_bytes;
    return HYENA_OK;
}

int hyena_conv_fwd_long_ex(const void *q, const void *k, const void *v, const void *h, int64_t B, int64_t L,
                           int64_t D, int64_t group_size, int64_t l_h, void *out, int dtype, void *workspace,
                           int64_t workspace_bytes, int reuse_spectra, void *stream) {
    FftPlan pl;
    int st = fft_plan(B, L, D, group_size, l_h, dtype, &pl);
    if (st != HYENA_OK) return st;
    if (reuse_spectra != 0 && reuse_spectra != 1) return HYENA_ERR_SHAPE;
    if (B == 0 || L == 0 || D == 0) return HYENA_OK;
    if (!q || !k || !v || (!h && !reuse_spectra) || !out) return HYENA_ERR_NULL;
    if (!workspace || workspace_bytes < pl.ws_bytes) return HYENA_ERR_WORKSPACE;
    const size_t eb = dtype == HYENA_DTYPE_F32 ? 4 : 2;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)workspace) & 15u)
        return HYENA_ERR_ALIGN;
    if ((uintptr_t)h & (eb - 1)) return HYENA_ERR_ALIGN;
    const size_t nbytes = (size_t)B * (size_t)L * (size_t)D * eb;
    const size_t hbytes = h ? (size_t)(D / group_size) * (size_t)l_h * eb : 0;
    const size_t wbytes = (size_t)pl.ws_bytes;
    if (overlaps(out, nbytes, q, nbytes) || overlaps(out, nbytes, k, nbytes) || overlaps(out, nbytes, v, nbytes) ||
        overlaps(out, nbytes, h, hbytes) || overlaps(workspace, wbytes, q, nbytes) ||
        overlaps(workspace, wbytes, k, nbytes) || overlaps(workspace, wbytes, v, nbytes) ||
        overlaps(workspace, wbytes, h, hbytes) || overlaps(workspace, wbytes, out, nbytes))
        return HYENA_ERR_ALIAS;

    const int64_t G = D / group_size;
    FftParams p = {};
    p.q = q; p.k = k; p.v = v; p.h = h; p.y = out;
    p.hs = (float2 *)workspace;
    p.ws = (float2 *)((char *)workspace + pl.hs_bytes);
    p.D = (int32_t)D;
    p.G = (int32_t)G;
    p.Gp = (int32_t)(G + (G & 1));
    p.group_size = (int32_t)group_size;
    p.l_h = (int32_t)l_h;
    p.N1 = pl.N1; p.N2 = pl.N2; p.log1 = pl.log1; p.log2 = pl.log2;
    p.N3 = pl.N3; p.log3 = pl.log3;
    const bool f32 = dtype == HYENA_DTYPE_F32;
    hipStream_t s = (hipStream_t)stream;

    auto launch = [&](const void *fn, const FftParams &q_, int P, int64_t units, int64_t nb, int lds) -> int {
        return fft_launch(fn, q_, P, units, nb, lds, s);
    };
    const int64_t M = (int64_t)pl.N2 * pl.N3;  // columns
    const int64_t cols = M / 2 + 1;
    const void *rows_seq, *rows_flt, *out_fn;
    const bool direct_filters = G <= kFftDirectFilters;
    if (pl.three) {
        rows_seq = rows3_kernel<0>(f32, pl.reg_rows3);
        rows_flt = direct_filters ? rows3_kernel<2>(f32, pl.reg_rows3) : rows3_kernel<1>(f32, pl.reg_rows3);
        out_fn = out3_kernel<0>(f32, pl.reg_rows3);
    } else {
        rows_seq = rows_kernel<0>(f32, pl.reg_rows);
        rows_flt = direct_filters ? rows_kernel<2>(f32, pl.reg_rows) : rows_kernel<1>(f32, pl.reg_rows);
        out_fn = out_kernel<0>(f32, pl.reg_rows);
    }
    // units per batch row of the row and output kernels: t1 (x t2 when three-level)
    const int64_t row_units = pl.three ? (int64_t)pl.N1 * pl.N2 : pl.N1;
    const int64_t mid_units = (int64_t)pl.N1 * pl.N3;

    // filter spectra: the filters as one sequence of G channels, min(l_h, L)
    // rows (kept from an earlier call when the caller says so)
    if (!reuse_spectra) {
        FftParams ph = p;
        ph.L = l_h < L ? l_h : L;
        ph.np = p.Gp / 2;
        if (!direct_filters) {
            st = transpose_filters(h, f32, p.G, p.Gp, l_h, ph.L, p.hs, s);
            ph.h = p.hs;  // [taps][Gp] fp32, in the spectra's place until the column pass writes them
        }
        if (st == HYENA_OK) st = launch(rows_flt, ph, pl.P_rows, row_units, 1, pl.lds_rows);
        if (st == HYENA_OK && pl.three)
            st = launch(mid_kernel<false>(pl.reg_mid), ph, pl.P_mid, mid_units, 1, pl.lds_mid);
        if (st == HYENA_OK) st = launch((const void *)fft_cols_kernel<0>, ph, pl.P_cols, cols, 1, pl.lds_cols);
    }
    // the sequence
    p.L = L;
    p.np = (int32_t)(D / 2);
    if (st == HYENA_OK) st = launch(rows_seq, p, pl.P_rows, row_units, B, pl.lds_rows);
    if (st == HYENA_OK && pl.three)
        st = launch(mid_kernel<false>(pl.reg_mid), p, pl.P_mid, mid_units, B, pl.lds_mid);
    // channel pairs inside one group (even group size): single columns
    if (st == HYENA_OK)
        st = group_size % 2 == 0 ? launch(col1_kernel(pl.reg_col1, pl.log1), p, pl.P_col1, M, B, pl.lds_col1)
                                 : launch((const void *)fft_cols_kernel<1>, p, pl.P_cols, cols, B, pl.lds_cols);
    if (st == HYENA_OK && pl.three)
        st = launch(mid_kernel<true>(pl.reg_mid), p, pl.P_mid, mid_units, B, pl.lds_mid);
    if (st == HYENA_OK) st = launch(out_fn, p, pl.P_rows, row_units, B, pl.lds_rows);
    if (st != HYENA_OK) return st;
    if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
    return HYENA_OK;
}

int hyena_conv_fwd_long(const void *q, const void *k, const void *v, const void *h, int64_t B, int64_t L,
                        int64_t D, int64_t group_size, int64_t l_h, void *out, int dtype, void *workspace,
                        int64_t workspace_bytes, void *stream) {
    return hyena_conv_fwd_long_ex(q, k, v, h, B, L, D, group_size, l_h, out, dtype, workspace, workspace_bytes, 0,
                                  stream);
}

int hyena_conv_bwd_long_workspace(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, int dtype,
                                  int64_t *bytes_out) {
    FftPlan pl;
    int st = fft_plan(B, L, D, group_size, l_h, dtype, &pl);
    if (st == HYENA_OK) st = fft_bwd_plan(B, D, group_size, &pl);
    if (st != HYENA_OK) return st;
    if (bytes_out) *bytes_out = (B == 0 || L == 0 || D == 0) ? 0 : pl.bwd_ws_bytes;
    return HYENA_OK;
}

int hyena_conv_bwd_long_ex(const void *q, const void *k, const void *v, const void *h, const void *dy, int64_t B,
                           int64_t L, int64_t D, int64_t group_size, int64_t l_h, void *dq, void *dk, void *dv,
                           float *dh, int dtype, void *workspace, int64_t workspace_bytes, int reuse_spectra,
                           void *stream) {
    FftPlan pl;
    int st = fft_plan(B, L, D, group_size, l_h, dtype, &pl);
    if (st == HYENA_OK) st = fft_bwd_plan(B, D, group_size, &pl);
    if (st != HYENA_OK) return st;
    if (reuse_spectra != 0 && reuse_spectra != 1) return HYENA_ERR_SHAPE;
    if (!q || !k || !v || (!h && !reuse_spectra) || !dy) return HYENA_ERR_NULL;
    if ((dk == nullptr) != (dv == nullptr)) return HYENA_ERR_NULL;
    const size_t eb = dtype == HYENA_DTYPE_F32 ? 4 : 2;
    uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)dy | (uintptr_t)workspace;
    if (dq) mis |= (uintptr_t)dq;
    if (dk) mis |= (uintptr_t)dk | (uintptr_t)dv;
    if (mis & 15u) return HYENA_ERR_ALIGN;
    if (((uintptr_t)h & (eb - 1)) || ((uintptr_t)dh & 3u)) return HYENA_ERR_ALIGN;
    const int64_t G = D / group_size;
    const bool empty = B == 0 || L == 0 || D == 0;
    const size_t nbytes = (size_t)B * (size_t)L * (size_t)D * eb;
    const size_t hbytes = h ? (size_t)G * (size_t)l_h * eb : 0;
    const size_t dhbytes = (size_t)G * (size_t)l_h * sizeof(float);
    const size_t wbytes = empty ? 0 : (size_t)pl.bwd_ws_bytes;
    // every output and the workspace are disjoint from every input and from each other
    const void *in[5] = {q, k, v, dy, h};
    const size_t in_n[5] = {nbytes, nbytes, nbytes, nbytes, hbytes};
    const void *outs[5] = {dq, dk, dv, dh, empty ? nullptr : workspace};
    const size_t out_n[5] = {nbytes, nbytes, nbytes, dhbytes, wbytes};
    for (int i = 0; i < 5; ++i) {
        if (!outs[i]) continue;
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], out_n[i], in[j], in_n[j])) return HYENA_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (outs[j] && overlaps(outs[i], out_n[i], outs[j], out_n[j])) return HYENA_ERR_ALIAS;
    }
    hipStream_t s = (hipStream_t)stream;
    const int64_t taps = l_h < L ? l_h : L;
    // the zero-fill and transpose grids
    if (dh && ((G * l_h + 255) / 256 > INT32_MAX || ((l_h + 63) / 64) * ((G + 63) / 64) > INT32_MAX))
        return HYENA_ERR_UNSUPPORTED;
    if (empty || (!dq && !dk && !dh)) {
        // no rows: dh is zero (D == 0: dh has no elements)
        if (dh && G * l_h > 0) {
            hipLaunchKernelGGL(fft_dh_tail_kernel, dim3((unsigned)((G * l_h + 255) / 256)), dim3(256), 0, s, dh, G,
                               l_h, (int64_t)0);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        }
        return HYENA_OK;
    }
    if (!workspace || workspace_bytes < pl.bwd_ws_bytes) return HYENA_ERR_WORKSPACE;

    FftParams p = {};
    p.h = h;
    p.hs = (float2 *)workspace;
    p.ws = (float2 *)((char *)workspace + pl.hs_bytes);
    p.D = (int32_t)D;
    p.G = (int32_t)G;
    p.Gp = (int32_t)(G + (G & 1));
    p.group_size = (int32_t)group_size;
    p.l_h = (int32_t)l_h;
    p.N1 = pl.N1; p.N2 = pl.N2; p.log1 = pl.log1; p.log2 = pl.log2;
    p.N3 = pl.N3; p.log3 = pl.log3;
    p.nb = (int32_t)B;
    const bool f32 = dtype == HYENA_DTYPE_F32;
    auto launch = [&](const void *fn, const FftParams &q_, int P, int64_t units, int64_t nb, int lds) -> int {
        return fft_launch(fn, q_, P, units, nb, lds, s);
    };
    const int64_t M = (int64_t)pl.N2 * pl.N3;
    const int64_t cols = M / 2 + 1;
    const int64_t row_units = pl.three ? (int64_t)pl.N1 * pl.N2 : pl.N1;
    const int64_t mid_units = (int64_t)pl.N1 * pl.N3;
    const void *rows_seq, *rows_flt;
    const bool direct_filters = G <= kFftDirectFilters;
    if (pl.three) {
        rows_seq = rows3_kernel<0>(f32, pl.reg_rows3);
        rows_flt = direct_filters ? rows3_kernel<2>(f32, pl.reg_rows3) : rows3_kernel<1>(f32, pl.reg_rows3);
    } else {
        rows_seq = rows_kernel<0>(f32, pl.reg_rows);
        rows_flt = direct_filters ? rows_kernel<2>(f32, pl.reg_rows) : rows_kernel<1>(f32, pl.reg_rows);
    }
    // the last inverse pass with each output form
    auto out_fn = [&](int mode) -> const void * {
        if (pl.three) {
            if (mode == 0) return out3_kernel<0>(f32, pl.reg_rows3);
            if (mode == 1) return out3_kernel<1>(f32, pl.reg_rows3);
            return out3_kernel<2>(true, pl.reg_rows3);
        }
        if (mode == 0) return out_kernel<0>(f32, pl.reg_rows);
        if (mode == 1) return out_kernel<1>(f32, pl.reg_rows);
        return out_kernel<2>(true, pl.reg_rows);
    };

    // filter spectra (the first work area serves as the filter pass's), or
    // kept in the workspace by an earlier call
    if (!reuse_spectra) {
        FftParams ph = p;
        ph.L = taps;
        ph.np = p.Gp / 2;
        if (!direct_filters) {
            st = transpose_filters(h, f32, p.G, p.Gp, l_h, taps, p.hs, s);
            ph.h = p.hs;  // [taps][Gp] fp32, in the spectra's place until the column pass writes them
        }
        if (st == HYENA_OK) st = launch(rows_flt, ph, pl.P_rows, row_units, 1, pl.lds_rows);
        if (st == HYENA_OK && pl.three)
            st = launch(mid_kernel<false>(pl.reg_mid), ph, pl.P_mid, mid_units, 1, pl.lds_mid);
        if (st == HYENA_OK) st = launch((const void *)fft_cols_kernel<0>, ph, pl.P_cols, cols, 1, pl.lds_cols);
    }
    p.L = L;
    p.np = (int32_t)(D / 2);
    float2 *area_dz = (float2 *)((char *)p.ws + pl.area_bytes);
    // x = k v into the first work area, dz = dy q into the second
    {
        FftParams px = p;
        px.k = k; px.v = v;
        if (st == HYENA_OK) st = launch(rows_seq, px, pl.P_rows, row_units, B, pl.lds_rows);
        FftParams pz = p;
        pz.k = dy; pz.v = q; pz.ws = area_dz;
        if (st == HYENA_OK) st = launch(rows_seq, pz, pl.P_rows, row_units, B, pl.lds_rows);
    }
    // the middle passes cover both work areas as 2B batch rows
    if (st == HYENA_OK && pl.three)
        st = launch(mid_kernel<false>(pl.reg_mid), p, pl.P_mid, mid_units, 2 * B, pl.lds_mid);
    {
        FftParams pc = p;
        pc.part = dh ? (float2 *)((char *)p.ws + 2 * pl.area_bytes) : nullptr;
        pc.n_slots = (int32_t)pl.n_slots;
        if (st == HYENA_OK)
            st = pl.bwd_col1 ? launch(bwd_col1_kernel(pl.reg_bwd1, pl.log1), pc, pl.P_bwd, M, B, pl.lds_bwd)
                             : launch((const void *)fft_bwd_cols_kernel, pc, pl.P_bwd, cols, B, pl.lds_bwd);
    }
    if (st == HYENA_OK && pl.three && (dq || dk))
        st = launch(mid_kernel<true>(pl.reg_mid), p, pl.P_mid, mid_units, 2 * B, pl.lds_mid);
    if (st == HYENA_OK && dq) {
        FftParams po = p;
        po.q = dy; po.y = dq;
        st = launch(out_fn(0), po, pl.P_rows, row_units, B, pl.lds_rows);
    }
    if (st == HYENA_OK && dk) {
        FftParams po = p;
        po.ws = area_dz; po.k = k; po.v = v; po.y = dk; po.y2 = dv;
        st = launch(out_fn(1), po, pl.P_rows, row_units, B, pl.lds_rows);
    }
    if (st == HYENA_OK && dh) {
        // group spectra -> one-row work area of Gp/2 group pairs (the first
        // work area, free once dq is out) -> inverse along f2 -> [taps][Gp]
        // in the second work area (free once dk and dv are out; B N D / 2
        // complex values >= taps Gp floats) -> dh [G][l_h]
        FftParams pd = p;
        pd.part = (float2 *)((char *)p.ws + 2 * pl.area_bytes);
        pd.np = p.Gp / 2;
        pd.nb = (int32_t)B;
        pd.pb_log = 0;
        while ((1 << pd.pb_log) < pl.P_bwd) ++pd.pb_log;
        pd.pb_tiles = (int32_t)pl.pb_tiles;
        pd.n_slots = (int32_t)pl.n_slots;
        pd.part_slot_major = pl.bwd_col1 ? 1 : 0;
        st = launch((const void *)fft_dh_cols_kernel, pd, pl.P_dh, cols, 1, pl.lds_dh);
        pd.L = taps;
        pd.y = area_dz;
        if (st == HYENA_OK && pl.three)
            st = launch(mid_kernel<true>(pl.reg_mid), pd, pl.P_mid, mid_units, 1, pl.lds_mid);
        if (st == HYENA_OK) st = launch(out_fn(2), pd, pl.P_rows, row_units, 1, pl.lds_rows);
        if (st == HYENA_OK) {
            const int64_t n_tblk = (l_h + 63) / 64, n_gblk = (G + 63) / 64;
            hipLaunchKernelGGL(fft_dh_transpose_kernel, dim3((unsigned)(n_tblk * n_gblk)), dim3(256), 0, s,
                               (const float *)area_dz, dh, (int)G, (int)p.Gp, (int)l_h, (int)taps, (int)n_tblk);
        }
    }
    if (st != HYENA_OK) return st;
    if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
    return HYENA_OK;
}

int hyena_conv_bwd_long(const void *q, const void *k, const void *v, const void *h, const void *dy, int64_t B,
                        int64_t L, int64_t D, int64_t group_size, int64_t l_h, void *dq, void *dk, void *dv,
                        float *dh, int dtype, void *workspace, int64_t workspace_bytes, void *stream) {
    return hyena_conv_bwd_long_ex(q, k, v, h, dy, B, L, D, group_size, l_h, dq, dk, dv, dh, dtype, workspace,
                                  workspace_bytes, 0, stream);
}

}  // extern "C"
