// Streaming reference for the benchmark (not part of the operator's ABI):
//     y = q * k * v   (bf16 in, fp32 products, bf16 out, round to nearest even)
// over [B, L, D] tensors, with access patterns of the grouped forward kernels
// in hyena_conv.hip and none of their arithmetic or on-chip staging:
//   * a workgroup owns one row segment of SEG bytes (256: the slab of an
//     8-wave forward workgroup; 512: a 16-wave one; 1024) and a span of
//     4 or 8 chunks of 64 rows of one batch row;
//   * every lane moves 16 bytes per access, through buffer loads with the
//     non-temporal policy, and stores with non-temporal, system-scope policy
//     (the forward kernel's store policy);
//   * PF chunks of q, k and v are in flight in registers, and the walk over
//     the span is unrolled at compile time;
//   * the grid runs slabs fastest (as the forward) or spans fastest.
// It reads three tensors and writes one, the operator's 8 bytes per
// token*channel, so its best rate is what the memory system gives that
// traffic: the attainable ceiling the forward kernels are measured against.
//
// C entry points (declared here only; the benchmark loads them with ctypes):
//   int hyena_stream_configs(void);                  number of patterns
//   int hyena_stream_config(int i, int *out6);       waves, SEG, span, PF, order, 0
//   int hyena_stream_read3_write1(int i, const void *q, const void *k,
//                                 const void *v, void *y, int64_t B,
//                                 int64_t L, int64_t D, void *stream);
// q, k, v, y are bf16 device pointers, 16-byte aligned, D * 2 a multiple of
// 16.  Returns 0, -1 for bad arguments, -8 if the launch failed.  Enqueued on
// `stream`, not waited for.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kRows = 64;      // rows per chunk
constexpr int kLoadPolicy = 2;    // nt
constexpr int kStorePolicy = 19;  // nt, sc0, sc1
constexpr uint32_t kOOB = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// two bf16 lanes of each operand: the product of the three, rounded once
__device__ inline uint32_t mul3(uint32_t a, uint32_t b, uint32_t c) {
    const float lo = __uint_as_float(a << 16) * __uint_as_float(b << 16) * __uint_as_float(c << 16);
    const float hi = __uint_as_float(a & 0xffff0000u) * __uint_as_float(b & 0xffff0000u) *
                     __uint_as_float(c & 0xffff0000u);
    const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

template <int NW, int SEG, int S, int PF, int ORD>
__global__ __launch_bounds__(64 * NW) void stream_read3_write1_kernel(const void *q, const void *k, const void *v,
                                                                      void *y, int64_t L, int D, int n_spans,
                                                                      int n_slabs) {
    constexpr int TPR = SEG / 16;          // lanes per row
    constexpr int RPL = 64 * NW / TPR;     // rows per access
    constexpr int NLD = kRows / RPL;       // accesses per tensor per chunk
    static_assert(NLD * RPL == kRows, "accesses must tile the chunk");

    int bid = blockIdx.x;
    const int per_b = n_spans * n_slabs;
    const int b = bid / per_b;
    bid -= b * per_b;
    const int slab = ORD == 0 ? bid % n_slabs : bid / n_spans;
    const int spn = ORD == 0 ? bid / n_slabs : bid % n_spans;
    const int64_t t0 = (int64_t)spn * S * kRows;
    const int64_t t1 = min(L, t0 + (int64_t)S * kRows);
    const int row_bytes = D * 2;
    const int c_off = slab * SEG;
    const size_t base = ((size_t)b * (size_t)L + (size_t)t0) * (size_t)row_bytes + (size_t)c_off;
    // the window ends at row t1 and channel D: everything past it reads 0 and is not written
    const uint32_t nrec = (uint32_t)((t1 - t0) * row_bytes - c_off);
    const __amdgpu_buffer_rsrc_t rq = rsrc((const char *)q + base, nrec);
    const __amdgpu_buffer_rsrc_t rk = rsrc((const char *)k + base, nrec);
    const __amdgpu_buffer_rsrc_t rv = rsrc((const char *)v + base, nrec);
    const __amdgpu_buffer_rsrc_t ry = rsrc((char *)y + base, nrec);

    const int tid = threadIdx.x;
    const int ld_row = tid / TPR;
    const int ld_seg = tid % TPR;
    const bool seg_ok = c_off + ld_seg * 16 < row_bytes;
    auto off = [&](int c, int i) -> uint32_t {
        return seg_ok ? (uint32_t)((c * kRows + i * RPL + ld_row) * row_bytes + ld_seg * 16) : kOOB;
    };

    u32x4_t qr[PF][NLD], kr[PF][NLD], vr[PF][NLD];
    auto load = [&](int c, int s) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            qr[s][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off(c, i), 0, kLoadPolicy));
            kr[s][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, off(c, i), 0, kLoadPolicy));
            vr[s][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off(c, i), 0, kLoadPolicy));
        }
    };
#pragma unroll
    for (int s = 0; s < PF; ++s) load(s, s);
#pragma unroll
    for (int c = 0; c < S; ++c) {
        const int s = c % PF;
        u32x4_t yv[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) yv[i][e] = mul3(qr[s][i][e], kr[s][i][e], vr[s][i][e]);
        if (c + PF < S) load(c + PF, s);
#pragma unroll
        for (int i = 0; i < NLD; ++i) __builtin_amdgcn_raw_buffer_store_b128(yv[i], ry, off(c, i), 0, kStorePolicy);
    }
}

typedef void (*StreamFn)(const void *, const void *, const void *, void *, int64_t, int, int, int);
struct Config {
    int waves, seg, span, pf, order;
    StreamFn fn;
};
#define CFG(NW, SEG, S, PF, ORD) {NW, SEG, S, PF, ORD, stream_read3_write1_kernel<NW, SEG, S, PF, ORD>}
// The grouped forward kernels' patterns, then the fastest ones a sweep of
// waves, SEG, span, PF and order found on MI355X at B=1, L=8192, D=4096.
const Config kConfigs[] = {
    CFG(8, 256, 8, 2, 0), CFG(16, 512, 8, 1, 0), CFG(16, 512, 8, 2, 0),
    CFG(16, 512, 4, 2, 0), CFG(8, 1024, 4, 1, 1), CFG(16, 512, 8, 3, 0),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

}  // namespace

extern "C" int hyena_stream_configs(void) { return kNumConfigs; }

extern "C" int hyena_stream_config(int i, int *out6) {
    if (i < 0 || i >= kNumConfigs || !out6) return -1;
    const Config &c = kConfigs[i];
    out6[0] = c.waves; out6[1] = c.seg; out6[2] = c.span; out6[3] = c.pf; out6[4] = c.order; out6[5] = 0;
    return 0;
}

extern "C" int hyena_stream_read3_write1(int i, const void *q, const void *k, const void *v, void *y, int64_t B,
                                         int64_t L, int64_t D, void *stream) {
    if (i < 0 || i >= kNumConfigs) return -1;
    const Config &c = kConfigs[i];
    if (!q || !k || !v || !y || B < 1 || L < 1 || D < 8 || (D * 2) % 16 != 0 || D > (1 << 28)) return -1;
    if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)y) & 15u) != 0) return -1;
    if ((int64_t)c.span * kRows * D * 2 >= ((int64_t)1 << 31)) return -1;  // 32-bit window offsets
    const int64_t n_spans = (L + c.span * kRows - 1) / (c.span * kRows);
    const int64_t n_slabs = (D * 2 + c.seg - 1) / c.seg;
    const int64_t grid = B * n_spans * n_slabs;
    if (grid > INT32_MAX || n_spans * n_slabs > INT32_MAX) return -1;
    hipLaunchKernelGGL(c.fn, dim3((unsigned)grid), dim3(64 * c.waves), 0, (hipStream_t)stream, q, k, v, y, L, (int)D,
                       (int)n_spans, (int)n_slabs);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}
