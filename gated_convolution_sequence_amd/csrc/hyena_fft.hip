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
// separated the same way), once per call.
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

struct FftParams {
    const void *q, *k, *v, *h;
    void *y;
    float2 *ws;          // [nb][N2][N1][np] complex work area
    float2 *hs;          // [N2][N1][Gp] filter spectra
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

// Global -> LDS staging of n values, kBatch per thread at a time: the loads
// of a batch are issued together (indices clamped into range, so none is
// conditional) and waited for once.
#ifndef HYENA_FFT_BATCH
#define HYENA_FFT_BATCH 8
#endif
constexpr int kBatch = HYENA_FFT_BATCH;
template <typename Load>
__device__ inline void stage_in(float2 *dst, int n, Load load) {
    for (int base = 0; base < n; base += kBatch * kFftThreads) {
        float2 r[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) r[u] = load(min(base + u * kFftThreads + (int)threadIdx.x, n - 1));
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = base + u * kFftThreads + (int)threadIdx.x;
            if (i < n) dst[i] = r[u];
        }
    }
}

// Input pair j at row t, zero past the end of the sequence or the pairs:
// (x[2j], x[2j+1]) with x = k v (SRC = 0, batch row b), or (h[2j][t],
// h[2j+1][t]) (SRC = 1, the filters; zero for a filter past the last).  The
// loads always go to a valid address (row 0, pair 0 when out of range) and
// the value is then replaced by zero.
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
    } else {
        const int g0 = 2 * jc, g1 = min(2 * jc + 1, p.G - 1);
        const size_t o0 = (size_t)g0 * p.l_h + tc, o1 = (size_t)g1 * p.l_h + tc;
        if constexpr (F32) {
            a = ((const float *)p.h)[o0];
            c = ((const float *)p.h)[o1];
        } else {
            a = __uint_as_float((uint32_t)((const uint16_t *)p.h)[o0] << 16);
            c = __uint_as_float((uint32_t)((const uint16_t *)p.h)[o1] << 16);
        }
        if (2 * jc + 1 >= p.G) c = 0.0f;
    }
    return ok ? make_float2(a, c) : make_float2(0.0f, 0.0f);
}

// Kernel 1: forward transform along t2 for one t1, then the twiddle.
// LDS (dynamic): two buffers of N2 P values, the N2 inner twiddles and the
// N2 inter-step twiddles W_N^(t1 f2) of this t1.
template <bool F32, int SRC>
__global__ __launch_bounds__(kFftThreads) void fft_rows_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int t1 = (item / p.n_tiles) % p.N1;
    const int b = item / (p.n_tiles * p.N1);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1, N2 = p.N2;
    const int NP = N2 << logP;
    const int64_t N = (int64_t)N1 * N2;
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + 2 * NP, *wt = tw + N2;
    stage_in(buf0, NP, [&](int i) {
        return load_pair<F32, SRC>(p, b, t1 + (int64_t)N1 * (i >> logP), (tile << logP) + (i & pmask));
    });
    fill_twiddles(tw, N2);
    for (int f2 = threadIdx.x; f2 < N2; f2 += kFftThreads) wt[f2] = twiddle(((int64_t)t1 * f2) & (N - 1), N);
    __syncthreads();
    const float2 *X = lds_fft(buf0, buf1, tw, N2, p.log2, logP, false);
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
// LDS (dynamic): two buffers of 2 N1 P values, the N1 inner twiddles and,
// per column, the N1 inter-step twiddles W_N^(-t1 f2).
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
    float2 *bufA = lds, *bufB = lds + NP2, *tw = lds + 2 * NP2;
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
    float2 *S = lds_fft(bufA, bufB, tw, N1, p.log1, lP2, false);
    float2 *Z = S == bufA ? bufB : bufA;
    // 2P divides the thread count, so a thread always has the same column
    // and channel pair: its filter spectra rows are fixed
    const int my_col = (threadIdx.x >> logP) & 1, my_pp = threadIdx.x & pmask;
    const int my_f2 = my_col ? fb : fa;
    const int my_j = (tile << logP) + my_pp;
    const int jc = min(my_j, p.np - 1);
    const float2 *hrow0 = p.hs + (size_t)my_f2 * N1 * p.Gp + (2 * jc) / p.group_size;
    const float2 *hrow1 = p.hs + (size_t)my_f2 * N1 * p.Gp + (2 * jc + 1) / p.group_size;
    for (int base = 0; base < NP2; base += kBatch * kFftThreads) {
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
                Z[i] = j < p.np ? make_float2(pu.x + pv.x, pu.y + pv.y) : make_float2(0.0f, 0.0f);
            }
        }
    }
    if constexpr (MODE == 1) {
        __syncthreads();
        const float2 *U = lds_fft(Z, S, tw, N1, p.log1, lP2, true);
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
// LDS (dynamic): two buffers of N1 P values, the N1 inner twiddles and the N1
// inter-step twiddles.
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
    float2 *bufA = lds, *bufB = lds + NP, *tw = lds + 2 * NP, *wt = tw + N1;
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
    float2 *S = lds_fft(bufA, bufB, tw, N1, p.log1, logP, false);
    float2 *Z = S == bufA ? bufB : bufA;
    // P divides the thread count, so a thread always has the same pair and
    // its filter spectrum row is fixed
    const int my_j = (tile << logP) + (threadIdx.x & pmask);
    const int jc = min(my_j, p.np - 1);
    const float2 *hrow = p.hs + (size_t)f2 * N1 * p.Gp + (2 * jc) / p.group_size;
    for (int base = 0; base < NP; base += kBatch * kFftThreads) {
        float2 hh[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int f1 = min(base + u * kFftThreads + (int)threadIdx.x, NP - 1) >> logP;
            hh[u] = hrow[(size_t)f1 * p.Gp];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = base + u * kFftThreads + (int)threadIdx.x;
            if (i >= NP) continue;
            Z[i] = my_j < p.np ? cmul(hh[u], S[i]) : make_float2(0.0f, 0.0f);
        }
    }
    __syncthreads();
    const float2 *U = lds_fft(Z, S, tw, N1, p.log1, logP, true);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        const int t1 = i >> logP;
        p.ws[(col0 + t1) * p.np + j] = cmul(U[i], wt[t1]);
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
// LDS (dynamic) of either: two buffers of N3 P (N2 P) values, the inner
// twiddles and the N3 (N2) inter-step twiddles.
template <bool F32, int SRC>
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
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + 2 * NP, *wt = tw + N3;
    stage_in(buf0, NP, [&](int i) {
        return load_pair<F32, SRC>(p, b, t1 + (int64_t)N1 * (t2 + (int64_t)N2 * (i >> logP)),
                                   (tile << logP) + (i & pmask));
    });
    fill_twiddles(tw, N3);
    for (int f3 = threadIdx.x; f3 < N3; f3 += kFftThreads) wt[f3] = twiddle(((int64_t)t2 * f3) & (M - 1), M);
    __syncthreads();
    const float2 *X = lds_fft(buf0, buf1, tw, N3, p.log3, logP, false);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int f3 = i >> logP;
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        p.ws[(((int64_t)b * M + (int64_t)f3 * N2 + t2) * N1 + t1) * p.np + j] = cmul(X[i], wt[f3]);
    }
}

template <bool INV>
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
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + 2 * NP, *wt = tw + N2;
    const int64_t row0 = (int64_t)b * M + (int64_t)f3 * N2;  // position of index 0 along t2 / f2
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
    const float2 *X = lds_fft(buf0, buf1, tw, N2, p.log2, logP, INV);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int u = i >> logP;
        const int j = (tile << logP) + (i & pmask);
        if (j >= p.np) continue;
        p.ws[((row0 + u) * N1 + t1) * p.np + j] = cmul(X[i], wt[u]);
    }
}

template <bool F32>
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
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + 2 * NP;
    stage_in(buf0, NP, [&](int i) {
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[(((int64_t)b * M + (int64_t)(i >> logP) * N2 + t2) * N1 + t1) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N3);
    __syncthreads();
    const float2 *z = lds_fft(buf0, buf1, tw, N3, p.log3, logP, true);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int t3 = i >> logP;
        const int j = (tile << logP) + (i & pmask);
        const int64_t t = t1 + (int64_t)N1 * (t2 + (int64_t)N2 * t3);
        if (j >= p.np || t >= p.L) continue;
        const size_t o = ((size_t)b * (size_t)p.L + (size_t)t) * (size_t)p.D + 2 * (size_t)j;
        const float z0 = z[i].x * scale, z1 = z[i].y * scale;
        if constexpr (F32) {
            const float2 qq = *(const float2 *)((const float *)p.q + o);
            *(float2 *)((float *)p.y + o) = make_float2(qq.x * z0, qq.y * z1);
        } else {
            const uint32_t qq = *(const uint32_t *)((const uint16_t *)p.q + o);
            const __bf16 y0 = (__bf16)(__uint_as_float(qq << 16) * z0);
            const __bf16 y1 = (__bf16)(__uint_as_float(qq & 0xffff0000u) * z1);
            *(uint32_t *)((uint16_t *)p.y + o) =
                (uint32_t)__builtin_bit_cast(uint16_t, y0) | ((uint32_t)__builtin_bit_cast(uint16_t, y1) << 16);
        }
    }
}

// Kernel 3: inverse transform along f2 for one t1, scale, gate, store.
// LDS (dynamic): two buffers of N2 P values and the N2 inner twiddles.
template <bool F32>
__global__ __launch_bounds__(kFftThreads) void fft_out_kernel(FftParams p) {
    extern __shared__ float2 lds[];
    const int item = xcd_item();
    const int tile = item % p.n_tiles;
    const int t1 = (item / p.n_tiles) % p.N1;
    const int b = item / (p.n_tiles * p.N1);
    const int logP = p.logP, pmask = (1 << logP) - 1, N1 = p.N1, N2 = p.N2;
    const int NP = N2 << logP;
    const float scale = 1.0f / ((float)N1 * (float)N2);
    float2 *buf0 = lds, *buf1 = lds + NP, *tw = lds + 2 * NP;
    stage_in(buf0, NP, [&](int i) {
        const int j = (tile << logP) + (i & pmask);
        const bool ok = j < p.np;
        const float2 v = p.ws[(((int64_t)b * N2 + (i >> logP)) * N1 + t1) * p.np + (ok ? j : 0)];
        return ok ? v : make_float2(0.0f, 0.0f);
    });
    fill_twiddles(tw, N2);
    __syncthreads();
    const float2 *z = lds_fft(buf0, buf1, tw, N2, p.log2, logP, true);
    for (int i = threadIdx.x; i < NP; i += kFftThreads) {
        const int t2 = i >> logP;
        const int j = (tile << logP) + (i & pmask);
        const int64_t t = t1 + (int64_t)N1 * t2;
        if (j >= p.np || t >= p.L) continue;
        const size_t o = ((size_t)b * (size_t)p.L + (size_t)t) * (size_t)p.D + 2 * (size_t)j;
        const float z0 = z[i].x * scale, z1 = z[i].y * scale;
        if constexpr (F32) {
            const float2 qq = *(const float2 *)((const float *)p.q + o);
            *(float2 *)((float *)p.y + o) = make_float2(qq.x * z0, qq.y * z1);
        } else {
            const uint32_t qq = *(const uint32_t *)((const uint16_t *)p.q + o);
            const __bf16 y0 = (__bf16)(__uint_as_float(qq << 16) * z0);
            const __bf16 y1 = (__bf16)(__uint_as_float(qq & 0xffff0000u) * z1);
            *(uint32_t *)((uint16_t *)p.y + o) =
                (uint32_t)__builtin_bit_cast(uint16_t, y0) | ((uint32_t)__builtin_bit_cast(uint16_t, y1) << 16);
        }
    }
}

struct FftPlan {
    int64_t N, ws_pairs, hs_bytes, ws_bytes;
    int N1, N2, N3, log1, log2, log3;
    bool three;                      // three-level split (N3 > 1)
    int P_rows, P_mid, P_cols, P_col1;          // pairs per workgroup: row (rows3/out3), middle,
    int lds_rows, lds_mid, lds_cols, lds_col1;  // column (paired, single) kernels; their LDS bytes
};

// Largest N done with the two-level split (columns of at most 256 points);
// above it the three-level split keeps every transform at 256 points or less.
constexpr int kFftTwoLevelMaxLogN = 16;

// Pairs per workgroup: LDS of about kFftBudget complex values (several
// workgroups per CU), at most 64 pairs, no more than the pairs there are; a
// single pair when even that exceeds the budget (the largest transforms).
#ifndef HYENA_FFT_BUDGET
#define HYENA_FFT_BUDGET 4096
#endif
constexpr int kFftBudget = HYENA_FFT_BUDGET;
#ifndef HYENA_FFT_COLS_BUDGET
#define HYENA_FFT_COLS_BUDGET HYENA_FFT_BUDGET
#endif
constexpr int kFftColsBudget = HYENA_FFT_COLS_BUDGET;  // the column kernel's
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
    pl->P_rows = pick_pairs(Mr, 2, pairs);
    pl->P_mid = pick_pairs(pl->N2, 2, pairs);
    pl->P_cols = pick_pairs(pl->N1, 4, pairs, kFftColsBudget);
    pl->lds_rows = (2 * Mr * pl->P_rows + 2 * Mr) * (int)sizeof(float2);
    pl->lds_mid = (2 * pl->N2 * pl->P_mid + 2 * pl->N2) * (int)sizeof(float2);
    pl->lds_cols = (4 * pl->N1 * pl->P_cols + 3 * pl->N1) * (int)sizeof(float2);
    pl->P_col1 = pick_pairs(pl->N1, 2, pairs);
    pl->lds_col1 = (2 * pl->N1 * pl->P_col1 + 2 * pl->N1) * (int)sizeof(float2);
    if (pl->lds_rows > kFftMaxLdsBytes || pl->lds_cols > kFftMaxLdsBytes || pl->lds_mid > kFftMaxLdsBytes ||
        pl->lds_col1 > kFftMaxLdsBytes)
        return HYENA_ERR_UNSUPPORTED;
    const int64_t Gp = G + (G & 1);
    pl->ws_pairs = B * (D / 2) > Gp / 2 ? B * (D / 2) : Gp / 2;
    pl->hs_bytes = pl->N * Gp * (int64_t)sizeof(float2);
    pl->ws_bytes = pl->N * pl->ws_pairs * (int64_t)sizeof(float2) + pl->hs_bytes;
    return HYENA_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
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

int hyena_conv_fwd_long(const void *q, const void *k, const void *v, const void *h, int64_t B, int64_t L,
                        int64_t D, int64_t group_size, int64_t l_h, void *out, int dtype, void *workspace,
                        int64_t workspace_bytes, void *stream) {
    FftPlan pl;
    int st = fft_plan(B, L, D, group_size, l_h, dtype, &pl);
    if (st != HYENA_OK) return st;
    if (B == 0 || L == 0 || D == 0) return HYENA_OK;
    if (!q || !k || !v || !h || !out) return HYENA_ERR_NULL;
    if (!workspace || workspace_bytes < pl.ws_bytes) return HYENA_ERR_WORKSPACE;
    const size_t eb = dtype == HYENA_DTYPE_F32 ? 4 : 2;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)workspace) & 15u)
        return HYENA_ERR_ALIGN;
    if ((uintptr_t)h & (eb - 1)) return HYENA_ERR_ALIGN;
    const size_t nbytes = (size_t)B * (size_t)L * (size_t)D * eb;
    const size_t hbytes = (size_t)(D / group_size) * (size_t)l_h * eb;
    const size_t wbytes = (size_t)pl.ws_bytes;
    if (overlaps(out, nbytes, q, nbytes) || overlaps(out, nbytes, k, nbytes) || overlaps(out, nbytes, v, nbytes) ||
        overlaps(out, nbytes, h, hbytes) || overlaps(workspace, wbytes, q, nbytes) ||
        overlaps(workspace, wbytes, k, nbytes) || overlaps(workspace, wbytes, v, nbytes) ||
        overlaps(workspace, wbytes, h, hbytes) || overlaps(workspace, wbytes, out, nbytes))
        return HYENA_ERR_ALIAS;

    const int64_t G = D / group_size;
    FftParams p;
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

    // One launch: pair tile, grid (batch rows x units x tiles), dynamic LDS.
    auto launch = [&](const void *fn, FftParams q_, int P, int64_t units, int64_t nb, int lds) -> int {
        q_.logP = 0;
        while ((1 << q_.logP) < P) ++q_.logP;
        q_.n_tiles = (q_.np + P - 1) / P;
        const int64_t grid = nb * units * q_.n_tiles;
        if (grid > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
        if (lds > 64 * 1024 &&
            hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
            return HYENA_ERR_LAUNCH;
        void *args[] = {&q_};
        if (hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kFftThreads), args, (size_t)lds, s) != hipSuccess)
            return HYENA_ERR_LAUNCH;
        return HYENA_OK;
    };
    const int64_t M = (int64_t)pl.N2 * pl.N3;  // columns
    const int64_t cols = M / 2 + 1;
    const void *rows_seq, *rows_flt, *out_fn;
    if (pl.three) {
        rows_seq = f32 ? (const void *)fft_rows3_kernel<true, 0> : (const void *)fft_rows3_kernel<false, 0>;
        rows_flt = f32 ? (const void *)fft_rows3_kernel<true, 1> : (const void *)fft_rows3_kernel<false, 1>;
        out_fn = f32 ? (const void *)fft_out3_kernel<true> : (const void *)fft_out3_kernel<false>;
    } else {
        rows_seq = f32 ? (const void *)fft_rows_kernel<true, 0> : (const void *)fft_rows_kernel<false, 0>;
        rows_flt = f32 ? (const void *)fft_rows_kernel<true, 1> : (const void *)fft_rows_kernel<false, 1>;
        out_fn = f32 ? (const void *)fft_out_kernel<true> : (const void *)fft_out_kernel<false>;
    }
    // units per batch row of the row and output kernels: t1 (x t2 when three-level)
    const int64_t row_units = pl.three ? (int64_t)pl.N1 * pl.N2 : pl.N1;
    const int64_t mid_units = (int64_t)pl.N1 * pl.N3;

    // filter spectra: the filters as one sequence of G channels, min(l_h, L) rows
    FftParams ph = p;
    ph.L = l_h < L ? l_h : L;
    ph.np = p.Gp / 2;
    st = launch(rows_flt, ph, pl.P_rows, row_units, 1, pl.lds_rows);
    if (st == HYENA_OK && pl.three)
        st = launch((const void *)fft_mid_kernel<false>, ph, pl.P_mid, mid_units, 1, pl.lds_mid);
    if (st == HYENA_OK) st = launch((const void *)fft_cols_kernel<0>, ph, pl.P_cols, cols, 1, pl.lds_cols);
    // the sequence
    p.L = L;
    p.np = (int32_t)(D / 2);
    if (st == HYENA_OK) st = launch(rows_seq, p, pl.P_rows, row_units, B, pl.lds_rows);
    if (st == HYENA_OK && pl.three)
        st = launch((const void *)fft_mid_kernel<false>, p, pl.P_mid, mid_units, B, pl.lds_mid);
    // channel pairs inside one group (even group size): single columns
    if (st == HYENA_OK)
        st = group_size % 2 == 0 ? launch((const void *)fft_col1_kernel, p, pl.P_col1, M, B, pl.lds_col1)
                                 : launch((const void *)fft_cols_kernel<1>, p, pl.P_cols, cols, B, pl.lds_cols);
    if (st == HYENA_OK && pl.three)
        st = launch((const void *)fft_mid_kernel<true>, p, pl.P_mid, mid_units, B, pl.lds_mid);
    if (st == HYENA_OK) st = launch(out_fn, p, pl.P_rows, row_units, B, pl.lds_rows);
    if (st != HYENA_OK) return st;
    if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
    return HYENA_OK;
}

}  // extern "C"
