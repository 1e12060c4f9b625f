// Streaming reference for the benchmark (not part of the operator's ABI):
//     y = q * k * v   (bf16 in, fp32 products, bf16 out, round to nearest even)
// over [B, L, D] tensors, with the access pattern of the grouped forward
// kernel in hyena_conv.hip and none of its arithmetic or on-chip staging:
//   * a workgroup owns one row segment of SEG bytes (256 or 512: the slab of
//     an 8- or a 16-wave forward workgroup) and a span of 8 chunks of 64 rows
//     of one batch row;
//   * every lane moves 16 bytes per access, through buffer loads with the
//     non-temporal policy, and stores with non-temporal, system-scope policy
//     (the forward kernel's store policy);
//   * two chunks of q, k and v are in flight in registers, and the walk over
//     the span is unrolled at compile time.
// It reads three tensors and writes one, the operator's 8 bytes per
// token*channel, so its rate is what the memory system gives that traffic
// pattern: the attainable ceiling the forward kernels are measured against.
//
// C entry point (declared here only; the benchmark loads it with ctypes):
//   int hyena_stream_read3_write1(const void *q, const void *k, const void *v,
//                                 void *y, int64_t B, int64_t L, int64_t D,
//                                 int seg_bytes, int waves, void *stream);
// seg_bytes is 256 or 512 and waves 8 or 16; q, k, v, y are bf16 device
// pointers, 16-byte aligned, D * 2 a multiple of 16.  Returns 0, -1 for bad
// arguments, -8 if the launch failed.  Enqueued on `stream`, not waited for.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kRows = 64;      // rows per chunk
constexpr int kSpan = 8;       // chunks per workgroup
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

template <int NW, int SEG>
__global__ __launch_bounds__(64 * NW) void stream_read3_write1_kernel(const void *q, const void *k, const void *v,
                                                                      void *y, int64_t L, int D, int n_spans,
                                                                      int n_slabs) {
    constexpr int TPR = SEG / 16;          // lanes per row
    constexpr int RPL = 64 * NW / TPR;     // rows per access
    constexpr int NLD = kRows / RPL;       // accesses per tensor per chunk
    constexpr int PF = 2;                  // chunks in flight
    static_assert(NLD * RPL == kRows, "accesses must tile the chunk");

    int bid = blockIdx.x;
    const int slab = bid % n_slabs;
    bid /= n_slabs;
    const int spn = bid % n_spans;
    const int b = bid / n_spans;
    const int64_t t0 = (int64_t)spn * kSpan * kRows;
    const int64_t t1 = min(L, t0 + (int64_t)kSpan * kRows);
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
    for (int c = 0; c < kSpan; ++c) {
        const int s = c % PF;
        u32x4_t yv[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) yv[i][e] = mul3(qr[s][i][e], kr[s][i][e], vr[s][i][e]);
        if (c + PF < kSpan) load(c + PF, s);
#pragma unroll
        for (int i = 0; i < NLD; ++i) __builtin_amdgcn_raw_buffer_store_b128(yv[i], ry, off(c, i), 0, kStorePolicy);
    }
}

}  // namespace

extern "C" int hyena_stream_read3_write1(const void *q, const void *k, const void *v, void *y, int64_t B,
                                         int64_t L, int64_t D, int seg_bytes, int waves, void *stream) {
    if (!q || !k || !v || !y || B < 1 || L < 1 || D < 8 || (D * 2) % 16 != 0 || D > (1 << 28)) return -1;
    if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)y) & 15u) != 0) return -1;
    if ((seg_bytes != 256 && seg_bytes != 512) || (waves != 8 && waves != 16)) return -1;
    if ((int64_t)kSpan * kRows * D * 2 >= ((int64_t)1 << 31)) return -1;  // 32-bit window offsets
    const int64_t n_spans = (L + kSpan * kRows - 1) / (kSpan * kRows);
    const int64_t n_slabs = (D * 2 + seg_bytes - 1) / seg_bytes;
    const int64_t grid = B * n_spans * n_slabs;
    if (grid > INT32_MAX || n_spans > INT32_MAX) return -1;
    void (*fn)(const void *, const void *, const void *, void *, int64_t, int, int, int) =
        waves == 8 ? (seg_bytes == 256 ? stream_read3_write1_kernel<8, 256> : stream_read3_write1_kernel<8, 512>)
                   : (seg_bytes == 256 ? stream_read3_write1_kernel<16, 256> : stream_read3_write1_kernel<16, 512>);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * waves), 0, (hipStream_t)stream, q, k, v, y, L, (int)D,
                       (int)n_spans, (int)n_slabs);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}
