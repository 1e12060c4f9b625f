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
//      FFT, twiddle W_N^(-t1 f2), write back in place;
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
// Inner transforms are radix-2 Stockham (self-sorting) in LDS with twiddles
// tabulated per workgroup; arithmetic is fp32 for both I/O types.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hyena_conv.h"

namespace {

constexpr int kFftThreads = 512;
constexpr int kFftLds = 8192;        // complex values per LDS buffer (64 KiB)
constexpr int kFftMaxM = 4096;       // largest inner transform
constexpr int kFftMaxLogN = 23;      // N <= 2^23

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
    int32_t P, n_tiles;  // pairs per workgroup, pair tiles
};

__device__ inline float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ inline float2 cconj(float2 a) { return make_float2(a.x, -a.y); }

// exp(-2 pi i m / n) for 0 <= m < n, n a power of two <= 2^23 (2m/n is
// exact in fp32, and sincospif reduces it exactly).
__device__ inline float2 twiddle(int64_t m, int64_t n) {
    float s, c;
    sincospif((float)(2 * m) / (float)n, &s, &c);
    return make_float2(c, -s);
}

// Twiddle table tw[m] = exp(-2 pi i m / M), m < M/2.
__device__ inline void fill_twiddles(float2 *tw, int M) {
    for (int m = threadIdx.x; m < M / 2; m += blockDim.x) tw[m] = twiddle(m, M);
}

// In-LDS M-point transform of P interleaved sequences (element j of
// sequence p at x[j P + p]), radix-2 Stockham: stage s combines
// sub-transforms of Ns = 2^s points into 2 Ns points,
//     y[(j - k) 2 + k] = a + w b,  y[(j - k) 2 + k + Ns] = a - w b,
// with a = x[j], b = x[j + M/2], k = j mod Ns, w = W_(2 Ns)^k (conjugated
// for the inverse).  Output in natural order; returns the buffer holding it.
// Callers synchronise before (x written) and the routine ends synchronised.
__device__ float2 *lds_fft(float2 *x, float2 *y, const float2 *tw, int M, int logM, int P, bool inverse) {
    const int half = M >> 1;
    const int n = half * P;
    for (int s = 0; s < logM; ++s) {
        const int Ns = 1 << s;
        const int tstride = half >> s;  // W_(2 Ns)^k = W_M^(k M / (2 Ns))
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int j = i / P;
            const int p = i - j * P;
            const int k = j & (Ns - 1);
            const float2 a = x[i];
            float2 w = tw[k * tstride];
            if (inverse) w.y = -w.y;
            const float2 b = cmul(x[i + n], w);
            const int d = ((j - k) << 1) + k;
            y[d * P + p] = make_float2(a.x + b.x, a.y + b.y);
            y[(d + Ns) * P + p] = make_float2(a.x - b.x, a.y - b.y);
        }
        __syncthreads();
        float2 *t = x;
        x = y;
        y = t;
    }
    return x;
}

// Input pair j at row t: (x[2j], x[2j+1]) with x = k v (SRC = 0, the
// sequence of batch row b) or (h[2j][t], h[2j+1][t]) (SRC = 1, the filters);
// zero past the end of either.
template <bool F32, int SRC>
__device__ inline float2 load_pair(const FftParams &p, int b, int64_t t, int j) {
    if (t >= p.L) return make_float2(0.0f, 0.0f);
    if constexpr (SRC == 0) {
        const size_t o = ((size_t)b * (size_t)p.L + (size_t)t) * (size_t)p.D + 2 * (size_t)j;
        if constexpr (F32) {
            const float2 kk = *(const float2 *)((const float *)p.k + o);
            const float2 vv = *(const float2 *)((const float *)p.v + o);
            return make_float2(kk.x * vv.x, kk.y * vv.y);
        } else {
            const uint32_t kk = *(const uint32_t *)((const uint16_t *)p.k + o);
            const uint32_t vv = *(const uint32_t *)((const uint16_t *)p.v + o);
            return make_float2(__uint_as_float(kk << 16) * __uint_as_float(vv << 16),
                               __uint_as_float(kk & 0xffff0000u) * __uint_as_float(vv & 0xffff0000u));
        }
    } else {
        const int g0 = 2 * j, g1 = 2 * j + 1;
        float a = 0.0f, c = 0.0f;
        if constexpr (F32) {
            a = ((const float *)p.h)[(size_t)g0 * p.l_h + t];
            if (g1 < p.G) c = ((const float *)p.h)[(size_t)g1 * p.l_h + t];
        } else {
            a = __uint_as_float((uint32_t)((const uint16_t *)p.h)[(size_t)g0 * p.l_h + t] << 16);
            if (g1 < p.G) c = __uint_as_float((uint32_t)((const uint16_t *)p.h)[(size_t)g1 * p.l_h + t] << 16);
        }
        return make_float2(a, c);
    }
}

// Kernel 1: forward transform along t2 for one t1, then the twiddle.
template <bool F32, int SRC>
__global__ __launch_bounds__(kFftThreads) void fft_rows_kernel(FftParams p) {
    __shared__ float2 buf[2][kFftLds];
    __shared__ float2 tw[kFftMaxM / 2];
    const int tile = blockIdx.x % p.n_tiles;
    const int t1 = (blockIdx.x / p.n_tiles) % p.N1;
    const int b = blockIdx.x / (p.n_tiles * p.N1);
    const int P = p.P, N1 = p.N1, N2 = p.N2;
    const int64_t N = (int64_t)N1 * N2;
    fill_twiddles(tw, N2);
    for (int i = threadIdx.x; i < N2 * P; i += blockDim.x) {
        const int t2 = i / P, pp = i - t2 * P;
        const int j = tile * P + pp;
        buf[0][i] = j < p.np ? load_pair<F32, SRC>(p, b, t1 + (int64_t)N1 * t2, j) : make_float2(0.0f, 0.0f);
    }
    __syncthreads();
    const float2 *X = lds_fft(buf[0], buf[1], tw, N2, p.log2, P, false);
    for (int i = threadIdx.x; i < N2 * P; i += blockDim.x) {
        const int f2 = i / P, pp = i - f2 * P;
        const int j = tile * P + pp;
        if (j >= p.np) continue;
        const float2 w = twiddle(((int64_t)t1 * f2) & (N - 1), N);
        p.ws[(((int64_t)b * N2 + f2) * N1 + t1) * p.np + j] = cmul(X[i], w);
    }
}

// Kernel 2: transforms along t1 for the column pair {f2, N2 - f2}.
// MODE 0 (filters): separate each pair's packed spectrum into the two
// filters' spectra and store them in hs.  MODE 1 (sequence): multiply by the
// filter spectra, inverse transform along f1, twiddle, store in place.
template <int MODE>
__global__ __launch_bounds__(kFftThreads) void fft_cols_kernel(FftParams p) {
    __shared__ float2 buf[4][kFftLds / 2];
    __shared__ float2 tw[kFftMaxM / 2];
    const int tile = blockIdx.x % p.n_tiles;
    const int c = (blockIdx.x / p.n_tiles) % (p.N2 / 2 + 1);
    const int b = blockIdx.x / (p.n_tiles * (p.N2 / 2 + 1));
    const int P = p.P, N1 = p.N1, N2 = p.N2;
    const int64_t N = (int64_t)N1 * N2;
    const int fa = c, fb = (N2 - c) & (N2 - 1);
    const bool self = fa == fb;
    const int ncol = self ? 1 : 2;
    fill_twiddles(tw, N1);
    for (int col = 0; col < ncol; ++col) {
        const int f2 = col ? fb : fa;
        for (int i = threadIdx.x; i < N1 * P; i += blockDim.x) {
            const int t1 = i / P, pp = i - t1 * P;
            const int j = tile * P + pp;
            buf[2 * col][i] = j < p.np ? p.ws[(((int64_t)b * N2 + f2) * N1 + t1) * p.np + j] : make_float2(0.0f, 0.0f);
        }
    }
    __syncthreads();
    float2 *S[2];
    S[0] = lds_fft(buf[0], buf[1], tw, N1, p.log1, P, false);
    S[1] = self ? S[0] : lds_fft(buf[2], buf[3], tw, N1, p.log1, P, false);
    // the other buffer of each pair receives the product
    float2 *Z[2] = {S[0] == buf[0] ? buf[1] : buf[0], S[1] == buf[2] ? buf[3] : buf[2]};
    for (int col = 0; col < ncol; ++col) {
        const int f2 = col ? fb : fa;
        const float2 *Sp = S[col], *Sm = S[col ^ (self ? 0 : 1)];
        for (int i = threadIdx.x; i < N1 * P; i += blockDim.x) {
            const int f1 = i / P, pp = i - f1 * P;
            const int j = tile * P + pp;
            // -(N2 f1 + f2) mod N = N2 f1m + (N2 - f2) mod N2: the partner column
            const int f1m = (N1 - f1 - (f2 > 0 ? 1 : 0)) & (N1 - 1);
            const float2 a = Sp[i];
            const float2 m = cconj(Sm[f1m * P + pp]);
            if constexpr (MODE == 0) {
                // filters 2j and 2j + 1: (a + m)/2 and (a - m)/(2i)
                if (j < p.np) {
                    const size_t o = ((size_t)f2 * N1 + f1) * p.Gp + 2 * (size_t)j;
                    p.hs[o] = make_float2(0.5f * (a.x + m.x), 0.5f * (a.y + m.y));
                    p.hs[o + 1] = make_float2(0.5f * (a.y - m.y), -0.5f * (a.x - m.x));
                }
            } else {
                float2 z = make_float2(0.0f, 0.0f);
                if (j < p.np) {
                    const int g0 = (2 * j) / p.group_size;
                    const int g1 = min(2 * j + 1, p.D - 1) / p.group_size;
                    const size_t o = ((size_t)f2 * N1 + f1) * p.Gp;
                    const float2 h0 = p.hs[o + g0];
                    if (g1 == g0) {
                        z = cmul(h0, a);
                    } else {
                        const float2 h1 = p.hs[o + g1];
                        const float2 s = make_float2(0.5f * (h0.x + h1.x), 0.5f * (h0.y + h1.y));
                        const float2 d = make_float2(0.5f * (h0.x - h1.x), 0.5f * (h0.y - h1.y));
                        const float2 u = cmul(s, a), v = cmul(d, m);
                        z = make_float2(u.x + v.x, u.y + v.y);
                    }
                }
                Z[col][i] = z;
            }
        }
    }
    if constexpr (MODE == 1) {
        __syncthreads();
        for (int col = 0; col < ncol; ++col) {
            const int f2 = col ? fb : fa;
            float2 *other = col ? (Z[1] == buf[2] ? buf[3] : buf[2]) : (Z[0] == buf[0] ? buf[1] : buf[0]);
            const float2 *U = lds_fft(Z[col], other, tw, N1, p.log1, P, true);
            for (int i = threadIdx.x; i < N1 * P; i += blockDim.x) {
                const int t1 = i / P, pp = i - t1 * P;
                const int j = tile * P + pp;
                if (j >= p.np) continue;
                const float2 w = cconj(twiddle(((int64_t)t1 * f2) & (N - 1), N));
                p.ws[(((int64_t)b * N2 + f2) * N1 + t1) * p.np + j] = cmul(U[i], w);
            }
        }
    }
}

// Kernel 3: inverse transform along f2 for one t1, scale, gate, store.
template <bool F32>
__global__ __launch_bounds__(kFftThreads) void fft_out_kernel(FftParams p) {
    __shared__ float2 buf[2][kFftLds];
    __shared__ float2 tw[kFftMaxM / 2];
    const int tile = blockIdx.x % p.n_tiles;
    const int t1 = (blockIdx.x / p.n_tiles) % p.N1;
    const int b = blockIdx.x / (p.n_tiles * p.N1);
    const int P = p.P, N1 = p.N1, N2 = p.N2;
    const float scale = 1.0f / ((float)N1 * (float)N2);
    fill_twiddles(tw, N2);
    for (int i = threadIdx.x; i < N2 * P; i += blockDim.x) {
        const int f2 = i / P, pp = i - f2 * P;
        const int j = tile * P + pp;
        buf[0][i] = j < p.np ? p.ws[(((int64_t)b * N2 + f2) * N1 + t1) * p.np + j] : make_float2(0.0f, 0.0f);
    }
    __syncthreads();
    const float2 *z = lds_fft(buf[0], buf[1], tw, N2, p.log2, P, true);
    for (int i = threadIdx.x; i < N2 * P; i += blockDim.x) {
        const int t2 = i / P, pp = i - t2 * P;
        const int j = tile * P + pp;
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
    int N1, N2, log1, log2, P;
};

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
    pl->log1 = (logN + 1) / 2;
    pl->log2 = logN / 2;
    pl->N1 = 1 << pl->log1;
    pl->N2 = 1 << pl->log2;
    // pairs per workgroup: the column kernel holds 4 buffers of N1 P values,
    // the row kernels 2 of N2 P
    int P = 64;
    while (P > 1 && (pl->N1 * P > kFftLds / 2 || pl->N2 * P > kFftLds)) P >>= 1;
    const int64_t pairs = D / 2;
    while (P > 1 && P / 2 >= pairs) P >>= 1;
    pl->P = P;
    const int64_t G = D / group_size;
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
    p.P = pl.P;
    const bool f32 = dtype == HYENA_DTYPE_F32;
    hipStream_t s = (hipStream_t)stream;

    // filter spectra: the filters as one sequence of G channels, l_h rows
    FftParams ph = p;
    ph.L = l_h < L ? l_h : L;
    ph.np = p.Gp / 2;
    ph.n_tiles = (ph.np + p.P - 1) / p.P;
    const int64_t g_rows = (int64_t)ph.n_tiles * pl.N1;
    const int64_t g_cols = (int64_t)ph.n_tiles * (pl.N2 / 2 + 1);
    if (f32) hipLaunchKernelGGL((fft_rows_kernel<true, 1>), dim3((unsigned)g_rows), dim3(kFftThreads), 0, s, ph);
    else hipLaunchKernelGGL((fft_rows_kernel<false, 1>), dim3((unsigned)g_rows), dim3(kFftThreads), 0, s, ph);
    hipLaunchKernelGGL((fft_cols_kernel<0>), dim3((unsigned)g_cols), dim3(kFftThreads), 0, s, ph);

    // the sequence
    p.L = L;
    p.np = (int32_t)(D / 2);
    p.n_tiles = (p.np + p.P - 1) / p.P;
    const int64_t rows = B * p.n_tiles * (int64_t)pl.N1;
    const int64_t cols = B * p.n_tiles * (int64_t)(pl.N2 / 2 + 1);
    if (rows > INT32_MAX || cols > INT32_MAX || g_rows > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
    if (f32) hipLaunchKernelGGL((fft_rows_kernel<true, 0>), dim3((unsigned)rows), dim3(kFftThreads), 0, s, p);
    else hipLaunchKernelGGL((fft_rows_kernel<false, 0>), dim3((unsigned)rows), dim3(kFftThreads), 0, s, p);
    hipLaunchKernelGGL((fft_cols_kernel<1>), dim3((unsigned)cols), dim3(kFftThreads), 0, s, p);
    if (f32) hipLaunchKernelGGL((fft_out_kernel<true>), dim3((unsigned)rows), dim3(kFftThreads), 0, s, p);
    else hipLaunchKernelGGL((fft_out_kernel<false>), dim3((unsigned)rows), dim3(kFftThreads), 0, s, p);
    if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
    return HYENA_OK;
}

}  // extern "C"
