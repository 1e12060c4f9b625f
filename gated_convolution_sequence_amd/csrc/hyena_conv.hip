// Hyena-SE / Hyena-MR for MI355X (gfx950):
//     y = q (.) (h * (k (.) v)),  grouped depthwise causal FIR, l_h <= 128,
// its backward, and for group sizes that are not a multiple of 16 the
// chunk-direction forward (or, for at most 8 taps, the direct forward).
// (Filters of any length: hyena_fft.hip.)
//
// Method (StripedHyena 2 explainer, page "04. hardware-aware convolution
// kernels"):
//   * section 1: the convolution is a product with a lower-triangular
//     Toeplitz matrix whose entry (row, column) is the tap h[row - column];
//   * section 3: split time into chunks of l_b rows; output chunk n is
//     H0 X_n + H1 X_{n-1} (+ H2 X_{n-2} once l_h > l_b + 1), X_{<0} = 0;
//   * section 4: the blocks are the same for every chunk and for every
//     channel of a group, so each group's products become dense GEMMs on the
//     matrix cores, with the blocks resident on chip; Algorithm 1 gates the
//     convolved chunk with q;
//   * section 6: the chunk direction is parallel (preload the blocks, load the
//     chunks, GEMM, write back);
//   * section 7: a Toeplitz tile is never stored in memory; each entry is
//     gathered from the filter by the difference of its row and column index.
//
// gfx950 mapping (l_b = 64 rows, one 16-channel group per wave):
//   * A workgroup of 8 waves owns a slab of 128 channels (8 groups of 16);
//     in bf16, 16 waves own 256 channels, so each row segment it reads is
//     512 bytes (HBM serves wider per-workgroup row segments faster): always
//     for filters of at most 33 taps, and for longer ones on grids of at
//     least 1024 workgroups.  It walks a span of consecutive 64-row chunks
//     of one batch row, plus the
//     32*KH rows before the span (the history its first chunks need), which
//     it reads last (see the walk order below).
//   * k and v arrive through 16-byte buffer loads, coalesced along channels;
//     x = k*v is formed in fp32, rounded to bf16 and written to an XOR-swizzled
//     LDS tile, which each wave re-reads time-major as the MFMA operand.
//   * Each wave computes Y^T (16 channels x 64 times) = X^T H^T with
//     v_mfma_f32_16x16x32_bf16: A = X^T (channel x input time), B = H^T
//     (input time x output time).  For an output tile of 16 rows and an input
//     step of 32 rows the Toeplitz operand depends only on their distance
//     e = nt - 2*kappa (in units of 16 rows), so a group needs 4 + 2*KH
//     distinct B fragments, built once per workgroup from the filter and kept
//     in registers.  Fragments whose taps all fall outside [0, l_h) are
//     skipped (the zero blocks of section 2).
//   * The previous chunks' X^T fragments stay in registers, so every input
//     row is read from HBM once per span.
//   * The epilogue stages the fp32 accumulators (4 consecutive channels per
//     lane) through a swizzled LDS tile, reads them row-major, multiplies by
//     q, rounds to bf16 and writes 16 bytes per lane.
//   * The 16-wave form for filters over 33 taps has no registers to keep
//     the B fragments or earlier chunks' fragments: it builds each B
//     fragment from a table of tap pairs in LDS right before the MFMAs that
//     use it, walks odd spans backwards in time, and gates its accumulators
//     in the MFMA layout (q read from LDS) before staging bf16 y.
//   * Buffer resources bound every access: rows before the batch start or
//     past the span, and channels past D, read as zero and are never
//     written.  That supplies X_{-1} = 0, ragged last chunks and partial slabs.
// The fp32 path has the same structure with v_mfma_f32_16x16x4_f32 (one
// input row per lane and step) and fp32 data in LDS.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "hyena_conv.h"

namespace {

#ifndef HYENA_WAVES
#define HYENA_WAVES 8
#endif
constexpr int kChunk = 64;               // l_b: rows per chunk
constexpr int kTile = 16;                // channels per wave (MFMA M)
constexpr int kWaves = HYENA_WAVES;      // waves per workgroup
constexpr int kSlab = kTile * kWaves;    // channels per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxTaps = 2 * kChunk;     // l_h <= 2 l_b
constexpr int kHOff = 64;                // filter staging: index = tap + kHOff
constexpr int kHLen = 256;               // staged taps per wave: [-64, 192)
constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every range
#ifndef HYENA_LOAD_POLICY
#define HYENA_LOAD_POLICY 2
#endif
#ifndef HYENA_STORE_POLICY
#define HYENA_STORE_POLICY 2
#endif
#ifndef HYENA_FWD_STORE_POLICY
#define HYENA_FWD_STORE_POLICY 19
#endif
// Cache-policy bits of the streaming buffer loads and stores (gfx950: 1 = sc0,
// 2 = nt, 16 = sc1).  Loads and stores are non-temporal.  The grouped forward
// kernel's stores add both scope bits (system scope), so that its written
// lines do not stay dirty in L2 for the next kernel to evict: at B=1,
// L=8192, D=4096 on MI355X an MR launch after another took 46.6-46.9 us
// against 47.4-47.7 us with nt alone (without nt, 51.2-51.4 us).  The same
// bits made the direct and chunk-direction kernels 3-4% slower.
constexpr int kLoadPolicy = HYENA_LOAD_POLICY;
constexpr int kStorePolicy = HYENA_STORE_POLICY;
constexpr int kFwdStorePolicy = HYENA_FWD_STORE_POLICY;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct Params {
    const void *q, *k, *v, *h;
    void *y;
    const void *kp, *vp; // rows before row 0 of each batch row ([B, P, D]), or null
    const void *g2;     // second gate (two-output form), or null
    void *y2;           // second output (two-output form), or null
    int64_t L;          // rows per batch
    int32_t D;          // channels (row pitch, elements)
    int32_t group_size;
    int32_t l_h;
    int32_t n_spans;    // spans per batch row
    int32_t n_slabs;    // channel slabs
    int32_t P;          // prefix rows in kp / vp (0: the history before row 0 is zero)
    int32_t span_blocks; // chunk-direction kernel: 256-row blocks per span
    int32_t span_rows;  // short-filter direct kernel: rows per span
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // Raw buffer (stride 0): an offset >= bytes reads 0 and drops writes.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int)bytes, 0x00020000);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t pack_bf16(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};  // round to nearest even
    return __builtin_bit_cast(uint32_t, r);
}

// Element-type traits: the I/O width and the LDS tile geometry.
// NW: waves per workgroup (one 16-channel tile each); the slab is 16 NW
// channels.
template <bool F32, int NW = kWaves> struct Tr;
template <int NW> struct Tr<false, NW> { // bf16 I/O
    static constexpr int EB = 2;         // bytes per element
    static constexpr int VEC = 8;        // elements per 16-byte access
    static constexpr int PITCH = kTile * NW * 2;     // LDS bytes per row
    static constexpr int TPR = PITCH / 16;           // threads per row (2 NW)
    static constexpr int RPL = 64 * NW / TPR;        // rows per load (32)
    static constexpr int NLD = kChunk / RPL;         // loads per tensor per chunk (2)
    // XOR swizzle of the 16-byte segment index by row (conflict-free
    // time-major reads of 16 channels x 4 row groups).
    __device__ static int swz(int row) { return ((row >> 3) & 3) << 1; }
    static_assert(NLD * RPL == kChunk, "loads must tile the chunk");
};
template <int NW> struct Tr<true, NW> {  // fp32 I/O
    static constexpr int EB = 4;
    static constexpr int VEC = 4;
    static constexpr int PITCH = kTile * NW * 4;
    static constexpr int TPR = PITCH / 16;           // 4 NW
    static constexpr int RPL = 64 * NW / TPR;        // 16
    static constexpr int NLD = kChunk / RPL;         // 4
    __device__ static int swz(int row) { return (row & 3) << 2; }
    static_assert(NLD * RPL == kChunk, "loads must tile the chunk");
};

// Matrix-core step of each element type: the MFMA operand fragment, the input
// rows one fragment covers (the MFMA K) and the fragments per 64-row chunk.
template <bool F32> struct Mma;
template <> struct Mma<false> {
    typedef bf16x8_t frag;               // v_mfma_f32_16x16x32_bf16: 8 rows per lane
    static constexpr int ROWS = 32;
    static constexpr int FPC = kChunk / ROWS;
};
template <> struct Mma<true> {
    typedef float frag;                  // v_mfma_f32_16x16x4_f32: 1 row per lane
    static constexpr int ROWS = 4;
    static constexpr int FPC = kChunk / ROWS;
};

// Staging buffers of the accumulator tile: two (each item's epilogue
// overlaps the next item's matrix-core work) from this many history steps,
// where registers already hold a CU to one workgroup; below, one, so that
// two workgroups still fit a CU's LDS.
#ifndef HYENA_ST2_MIN_KH
#define HYENA_ST2_MIN_KH 2
#endif


// Kernel: F32 selects the element type, KH the 32-row history steps
// (KH = ceil((l_h - 1) / 32)), PF the chunks of k, v and q kept in flight,
// S the chunks of one span.  The walk over the span is fully unrolled: the
// prefetched registers are then never loop-carried, so the compiler's
// memory-counter waits are exact and no in-flight load is copied.
//
// Walk order.  Chunk c of a span needs its own rows and the 32*KH rows
// before it, i.e. chunks c - H .. c (H history chunks before the span).  The
// rows two workgroups read -- the last H chunks of a span, which are the
// next span's history -- use the L2-allocating policy, so that whichever of
// the two reads comes second hits in L2.  Two walks place those reads:
//   * deferred (the kernels that keep their Toeplitz fragments in
//     registers): the span's own chunks first, computing each from chunk
//     ND on right after it is ingested; the first ND chunks need history,
//     so their operand fragments are kept and their outputs deferred.  The
//     history is ingested last, while the preceding span's workgroup (same
//     slab, same XCD under the round-robin dispatch, dispatched together)
//     reads the same rows as its own last chunks; then the deferred chunks.
//   * alternating (the 16-wave kernels that build fragments per use; no
//     registers to spare for deferred fragments): even spans walk up, the
//     history and then chunks 0 .. S-1, each computed right after it is
//     ingested; odd spans walk down, chunks S-1 .. 0 and then the history,
//     chunk c computed right after chunk c - H is ingested.  A shared chunk
//     is then read by both workgroups at the same point of their walks: at
//     the start of an odd span and of the even span after it, and at the end
//     of an even span and of the odd span after it.
// Every output tile sums its input steps in the same (ascending) order in
// either walk and direction, so the walk does not change a bit of the
// result.
//
// REV walks time backwards: logical row t is physical row L-1-t, so the same
// causal filter applied in the walk's order computes sum_s h[s] x[t+s] (the
// input gradient of the operator).  DUAL gates the one convolution with two
// tensors into two outputs (y = q acc, y2 = g2 acc).
template <bool F32, int KH, int PF, int S, bool REV = false, bool DUAL = false, int NW = kWaves>
__global__ __launch_bounds__(64 * NW) void hyena_fwd_kernel(Params p) {
    using T = Tr<F32, NW>;
    constexpr int SLAB = kTile * NW;                      // channels per workgroup
    using M = Mma<F32>;
    using frag = typename M::frag;
    constexpr int HROWS = 32 * KH;                        // history rows before a span
    constexpr int H = (HROWS + kChunk - 1) / kChunk;      // history chunks
    constexpr int NI = S + H;                             // ingested chunks
    constexpr int NH = HROWS / M::ROWS;                   // history fragments
    constexpr int NX = NH + M::FPC;                       // fragments one chunk reads
    constexpr int ST_PITCH = SLAB * 4;                    // fp32 staging row, bytes
    constexpr int kStBufs = KH >= HYENA_ST2_MIN_KH && NW == kWaves ? 2 : 1;

    // x = k*v of the current chunk (row-major, swizzled), the fp32
    // accumulators of the current chunk (and, with two staging buffers, of the
    // previous one; row-major, swizzled) and the filters.
    __shared__ __attribute__((aligned(16))) unsigned char xs[kChunk * T::PITCH];
    // 16-wave form with history (Toeplitz fragments built per use): the
    // gated output is staged instead of the accumulators (see gate below)
    constexpr bool GSTAGE = !F32 && NW > kWaves && KH >= 2;
    __shared__ __attribute__((aligned(16))) unsigned char st[GSTAGE ? 16 : kStBufs * kChunk * ST_PITCH];
    // (GSTAGE) q of the next compute item, and two tiles of gated output,
    // bf16 row-major with 16- and 8-byte units XOR-swizzled by row (gaddr)
    __shared__ __attribute__((aligned(16))) unsigned char qs[GSTAGE ? kChunk * T::PITCH : 16];
    __shared__ __attribute__((aligned(16))) unsigned char ys[GSTAGE ? 2 * kChunk * T::PITCH : 16];
    // the filter, zero outside [0, l_h): fp32 taps at index tap + kHOff, or
    // in bf16 pairs (h[t], h[t-1]) in one dword (low, high half) at index
    // kHLen - 1 - (t + kHOff), so that a Toeplitz fragment (8 taps
    // descending) is 4 dwords two entries apart at rising addresses, in
    // fragment order
    __shared__ std::conditional_t<F32, float, uint32_t> hs[NW][kHLen];

    const int tid = threadIdx.x;
    const int w = tid >> 6;           // wave = 16-channel tile of the slab
    const int l = tid & 63;
    const int n16 = l & 15;
    const int q4 = l >> 4;

    int bid = blockIdx.x;
    const int slab = bid % p.n_slabs;
    bid /= p.n_slabs;
    const int spn = bid % p.n_spans;
    const int b = bid / p.n_spans;
    // 16-wave form with history: Toeplitz fragments built per use, not kept
    constexpr bool FLY = !F32 && NW > kWaves && KH >= 2;
    // walk (see above): deferred for the kernels that keep their Toeplitz
    // fragments in registers, alternating for FLY
    constexpr int kWalk = FLY ? 1 : 0;
    const bool desc = kWalk == 1 && H > 0 && (spn & 1);
    constexpr int ND = kWalk != 0 ? 0 : (KH + 1) / 2 < S ? (KH + 1) / 2 : S;  // deferred chunks (walk 0)

    const int64_t t_begin = (int64_t)spn * S * kChunk;
    const int64_t t_stop = min(p.L, t_begin + (int64_t)S * kChunk);
    const int64_t base_row = max((int64_t)0, t_begin - HROWS);
    const int c_begin = slab * SLAB;
    const int row_bytes = p.D * T::EB;

    // Byte window [base, base + nrec) of this workgroup: rows base_row ..
    // t_stop-1 of batch b, starting at channel c_begin.  The host keeps it
    // below 2^31 bytes, so a negative (earlier) row offset is out of range,
    // as is every row at or past t_stop.
    // Under REV the window holds the same logical rows, at physical rows
    // L - t_stop .. L - 1 - base_row, in decreasing order.
    const int nwin = (int)(t_stop - base_row);
    const size_t first_phys = REV ? (size_t)(p.L - t_stop) : (size_t)base_row;
    const size_t base_off = ((size_t)b * (size_t)p.L + first_phys) * (size_t)row_bytes +
                            (size_t)c_begin * T::EB;
    const uint32_t nrec = (uint32_t)(nwin * row_bytes - c_begin * T::EB);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char *)p.q + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char *)p.k + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char *)p.v + base_off, nrec);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc((char *)p.y + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rg2 = make_rsrc(DUAL ? (const char *)p.g2 + base_off : (const char *)p.q, DUAL ? nrec : 0u);
    const __amdgpu_buffer_rsrc_t ry2 = make_rsrc(DUAL ? (char *)p.y2 + base_off : (char *)p.y, DUAL ? nrec : 0u);
    const int row0 = (int)(t_begin - base_row);       // window row of chunk 0
    // The caller's prefix rows (the P rows before row 0 of batch row b), read
    // instead of zeros by history chunks that lie before row 0.  With P = 0
    // the window is empty and every such read returns zero.
    const size_t pre_off = (size_t)b * (size_t)p.P * (size_t)row_bytes + (size_t)c_begin * T::EB;
    const uint32_t nrec_p = p.P > 0 ? (uint32_t)(p.P * row_bytes - c_begin * T::EB) : 0u;
    const __amdgpu_buffer_rsrc_t rkp = make_rsrc(p.P > 0 ? (const char *)p.kp + pre_off : (const char *)p.k, nrec_p);
    const __amdgpu_buffer_rsrc_t rvp = make_rsrc(p.P > 0 ? (const char *)p.vp + pre_off : (const char *)p.v, nrec_p);

    const bool tile_ok = c_begin + w * kTile < p.D;

    // ---- cooperative row-major access: thread -> (row, 16-byte segment) ----
    // q, k, v and y all use it: 16 bytes per lane, whole 256-byte rows.
    const int ld_row = tid / T::TPR;
    const int ld_seg = tid % T::TPR;
    const bool seg_ok = c_begin + ld_seg * T::VEC < p.D;
    const int ld_base = (REV ? -ld_row : ld_row) * row_bytes + ld_seg * 16;
    // Offset of chunk c (relative to the span start), load i.  Rows past the
    // span or before the history fall outside the byte window (no traffic,
    // no store); `need` = false sends the access outside it too.
    auto io_off = [&](int c, int i, bool need) -> uint32_t {
        const int lr = row0 + c * kChunk + i * T::RPL;  // logical window row (+ ld_row)
        const int r = (REV ? nwin - 1 - lr : lr) * row_bytes + ld_base;
        return (seg_ok && need) ? (uint32_t)r : kOOB;
    };
    constexpr int NG = DUAL ? 2 : 1;  // gates per row
    u32x4_t kr[PF][T::NLD], vr[PF][T::NLD], qr[PF][NG][T::NLD];

    // Load chunk c (relative to the span start; history chunks are
    // negative) of k and v.  The rows two workgroups read -- a span's last H
    // chunks, which are the next span's history -- use the default
    // (L2-allocating) policy, so that the second of the two reads hits in L2;
    // every other row is read once and streams past L2.  `need` = false
    // sends the access outside the window (no traffic).
    auto load_kv = [&](int c, bool need, u32x4_t *kd, u32x4_t *vd) {
        const bool keep = need && (c >= S - H || c < 0);
        // a chunk lies wholly before or wholly after row 0 (spans start on
        // chunk boundaries); before it, read the prefix rows P + t
        const int64_t t0c = t_begin + (int64_t)c * kChunk;
        const bool pre = need && t0c < 0;
        const __amdgpu_buffer_rsrc_t sk = pre ? rkp : rk;
        const __amdgpu_buffer_rsrc_t sv = pre ? rvp : rv;
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int rp = (int)(p.P + t0c) + i * T::RPL;
            const uint32_t o = pre ? (seg_ok ? (uint32_t)(rp * row_bytes + ld_base) : kOOB)
                                   : io_off(c, i, need);
            if (keep) {
                kd[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sk, o, 0, 0));
                vd[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sv, o, 0, 0));
            } else {
                kd[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sk, o, 0, kLoadPolicy));
                vd[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sv, o, 0, kLoadPolicy));
            }
        }
    };
    auto load_q = [&](int c, bool need, u32x4_t (*qd)[T::NLD]) {
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            qd[0][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, io_off(c, i, need), 0, kLoadPolicy));
            if constexpr (DUAL)
                qd[NG - 1][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rg2, io_off(c, i, need), 0, kLoadPolicy));
        }
    };
    // chunk of ingest item i and of compute item j
    auto ld_chunk = [&](int i) -> int {
        if constexpr (kWalk == 0) return i < S ? i : -H + (i - S);
        return desc ? S - 1 - i : i - H;
    };
    auto cp_chunk = [&](int j) -> int {
        if constexpr (kWalk == 0) return j < S - ND ? ND + j : j - (S - ND);
        return desc ? S - 1 - j : j;
    };
    // x = k*v for this thread's rows -> xs.
    auto store_x = [&](const u32x4_t *kd, const u32x4_t *vd) {
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int row = i * T::RPL + ld_row;
            u32x4_t xv;
            if constexpr (F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xv[e] = __float_as_uint(__uint_as_float(kd[i][e]) * __uint_as_float(vd[i][e]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xv[e] = pack_bf16(bf_lo(kd[i][e]) * bf_lo(vd[i][e]),
                                      bf_hi(kd[i][e]) * bf_hi(vd[i][e]));
            }
            *(u32x4_t *)(&xs[row * T::PITCH + ((ld_seg ^ T::swz(row)) << 4)]) = xv;
        }
    };
    // Accumulator staging: row t_out, 16-byte segment (4 fp32 channels) XOR
    // (row & 15), so 16 lanes writing one segment column of 16 rows, and the
    // row-major readers, hit distinct banks.
    auto st_addr = [&](int row, int seg) -> int { return row * ST_PITCH + ((seg ^ (row & 15)) << 4); };

    // Prologue: the first PF ingest items and the first PF compute items in
    // flight.  Each ingest then refills its slot with the item PF ahead, and
    // each compute the q slot with the compute item PF ahead.
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        load_kv(s < NI ? ld_chunk(s) : S, s < NI, kr[s], vr[s]);
        load_q(s < S ? cp_chunk(s) : S, s < S, qr[s]);
    }

    // ---- stage this wave's filter (zero outside [0, l_h)), after the first
    // chunks' loads are issued so that the two latencies overlap.  Every tap
    // load is issued unconditionally (an index outside the filter reads the
    // row's first tap, which is then replaced by zero), so all are in flight
    // together.
    {
        const int g = tile_ok ? (c_begin + w * kTile) / p.group_size : 0;
        const size_t hrow = (size_t)g * p.l_h;
        constexpr int NTL = kHLen / 64;  // staged entries per lane
        if constexpr (F32) {
            float hv[NTL];
#pragma unroll
            for (int j = 0; j < NTL; ++j) {
                const int tap = l + 64 * j - kHOff;
                hv[j] = ((const float *)p.h)[hrow + (tile_ok && tap >= 0 && tap < p.l_h ? tap : 0)];
            }
#pragma unroll
            for (int j = 0; j < NTL; ++j) {
                const int tap = l + 64 * j - kHOff;
                hs[w][l + 64 * j] = tile_ok && tap >= 0 && tap < p.l_h ? hv[j] : 0.0f;
            }
        } else {
            const uint16_t *hg = (const uint16_t *)p.h + hrow;
            uint32_t lo[NTL], hi[NTL];
#pragma unroll
            for (int j = 0; j < NTL; ++j) {
                const int tap = l + 64 * j - kHOff;
                lo[j] = hg[tile_ok && tap >= 0 && tap < p.l_h ? tap : 0];
                hi[j] = hg[tile_ok && tap >= 1 && tap <= p.l_h ? tap - 1 : 0];
            }
#pragma unroll
            for (int j = 0; j < NTL; ++j) {
                const int tap = l + 64 * j - kHOff;
                const uint32_t a = tile_ok && tap >= 0 && tap < p.l_h ? lo[j] : 0u;
                const uint32_t b = tile_ok && tap >= 1 && tap <= p.l_h ? hi[j] : 0u;
                hs[w][kHLen - 1 - (l + 64 * j)] = a | (b << 16);
            }
        }
    }

    __syncthreads();  // filters staged

    // ---- Toeplitz operand fragments and the time-major operand read --------
    // B = H^T: lane (n16 = output time within a 16-row tile, q4 = input-row
    // group), element j = input row.  The operand of output tile nt and input
    // step kappa depends only on their distance: bf16 e = nt - 2 kappa (units
    // of 16 rows), fp32 e4 = 4 nt - kappa (units of 4 rows).
    constexpr int NE = F32 ? 16 + NH : 4 + 2 * KH;
    frag F[FLY ? 1 : NE];
    // bf16 Toeplitz fragment e: element j = h[16 e + n16 - 8 q4 - j], i.e.
    // the pairs of taps 16 e + n16 - 8 q4 - 2 m, m = 0..3, which sit at
    // entries kHLen - 1 - kHOff - 16 e - n16 + 8 q4 + 2 m: one base per lane
    // (that of e = NE - 1, at least 0) and constant offsets
    const uint32_t *hbase = nullptr;
    if constexpr (!F32) hbase = &hs[w][kHLen - 1 - kHOff - 16 * (NE - 1) - n16 + 8 * q4];
    auto tap_frag = [&](int e) -> frag {
        if constexpr (F32) {
            return frag{};
        } else {
            const uint32_t *hw = hbase + 16 * (NE - 1 - e);
            const u32x4_t d = {hw[0], hw[2], hw[4], hw[6]};
            return __builtin_bit_cast(frag, d);
        }
    };
    const int ch = w * kTile + n16;
    int rd_base;
    if constexpr (F32) {
#pragma unroll
        for (int i = 0; i < NE; ++i) F[i] = hs[w][4 * (i - 3) + n16 - q4 + kHOff];
        rd_base = q4 * T::PITCH + ((((ch >> 2) ^ (4 * q4))) << 4) + ((ch & 3) << 2);
    } else {
        if constexpr (!FLY) {
#pragma unroll
            for (int e = 0; e < NE; ++e) F[e] = tap_frag(e);
        }
        // channel 16w + n16, rows 8 q4 + j (+ 32 kappa); their swizzle is 2 q4
        rd_base = (8 * q4) * T::PITCH + ((((ch >> 3) ^ (2 * q4))) << 4) + ((ch & 7) << 1);
    }
    // This chunk's FPC operand fragments from xs (A = X^T: lane n16 = channel).
    auto read_frags = [&](frag *dst) {
        if constexpr (F32) {
#pragma unroll
            for (int s4 = 0; s4 < M::FPC; ++s4)
                dst[s4] = *(const float *)(&xs[rd_base + (4 * s4) * T::PITCH]);
        } else {
#pragma unroll
            for (int kk = 0; kk < M::FPC; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    dst[kk][j] = __builtin_bit_cast(__bf16, *(const uint16_t *)(&xs[rd_base + (32 * kk + j) * T::PITCH]));
        }
    };
    // compute item j (chunk c) from its NX fragments Xc (history first):
    // the four 16-row output tiles into registers
    auto mma = [&](const frag *Xc, f32x4_t *acc) {
        if constexpr (FLY) {
            // e descending: for each output tile the input steps run in the
            // same (ascending) order as below
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            // each fragment is read while the previous one's MFMAs run
            frag fnext = tap_frag(NE - 1);
#pragma unroll
            for (int e = NE - 1; e >= 0; --e) {
                const frag fe = fnext;
                if (e > 0) fnext = tap_frag(e - 1);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if ((nt - e) % 2 != 0) continue;
                    const int kk = NH + (nt - e) / 2;  // e = nt - 2 (kk - NH)
                    if (kk < 0 || kk >= NX) continue;
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Xc[kk], fe, acc[nt], 0, 0, 0);
                }
            }
            return;
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NX; ++kk) {
                if constexpr (F32) {
                    const int e4 = 4 * nt - (kk - NH);
                    if (e4 < -3 || e4 + 3 >= NE) continue;
                    if (4 * e4 - 3 >= p.l_h) continue;  // every tap past the filter
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(Xc[kk], F[e4 + 3], acc[nt], 0, 0, 0);
                } else {
                    const int e = nt - 2 * (kk - NH);
                    if (e < 0) continue;  // strictly above the diagonal: all zero
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Xc[kk], F[e], acc[nt], 0, 0, 0);
                }
            }
        }
    };
    // the tiles of item j -> its staging buffer (lane: output time 16 nt +
    // n16, channels 4 q4 .. 4 q4 + 3)
    auto stage = [&](int j, const f32x4_t *acc) {
        unsigned char *sb = st + (j % kStBufs) * (kChunk * ST_PITCH);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) *(f32x4_t *)(&sb[st_addr(16 * nt + n16, 4 * w + q4)]) = acc[nt];
    };
    // epilogue of item j, once its staging buffer is complete: y = q * acc
    // (and y2 = g2 * acc) for this thread's rows, 16-byte stores.  LDS tiles
    // are in walk order; io_off maps the thread's walk row to its physical
    // row (REV: backwards) for the gate load and the store alike.
    auto finish = [&](int j) {
        const int c = cp_chunk(j);
        const unsigned char *sb = st + (j % kStBufs) * (kChunk * ST_PITCH);
        u32x4_t (*qd)[T::NLD] = qr[j % PF];
        u32x4_t yv[NG][T::NLD];
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int row = i * T::RPL + ld_row;
            f32x4_t a[2];
            if constexpr (F32) {
                a[0] = *(const f32x4_t *)(&sb[st_addr(row, ld_seg)]);
            } else {
                a[0] = *(const f32x4_t *)(&sb[st_addr(row, 2 * ld_seg)]);
                a[1] = *(const f32x4_t *)(&sb[st_addr(row, 2 * ld_seg + 1)]);
            }
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const u32x4_t gq = qd[gi][i];
                if constexpr (F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) yv[gi][i][e] = __float_as_uint(__uint_as_float(gq[e]) * a[0][e]);
                } else {
                    yv[gi][i][0] = pack_bf16(bf_lo(gq[0]) * a[0][0], bf_hi(gq[0]) * a[0][1]);
                    yv[gi][i][1] = pack_bf16(bf_lo(gq[1]) * a[0][2], bf_hi(gq[1]) * a[0][3]);
                    yv[gi][i][2] = pack_bf16(bf_lo(gq[2]) * a[1][0], bf_hi(gq[2]) * a[1][1]);
                    yv[gi][i][3] = pack_bf16(bf_lo(gq[3]) * a[1][2], bf_hi(gq[3]) * a[1][3]);
                }
            }
        }
        // refill q before storing y, so y never shares registers with q
        load_q(j + PF < S ? cp_chunk(j + PF) : S, j + PF < S, qd);
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            __builtin_amdgcn_raw_buffer_store_b128(yv[0][i], ry, io_off(c, i, true), 0, kFwdStorePolicy);
            if constexpr (DUAL)
                __builtin_amdgcn_raw_buffer_store_b128(yv[NG - 1][i], ry2, io_off(c, i, true), 0, kFwdStorePolicy);
        }
    };
    // ---- (GSTAGE) gated staging.  Two tiles of fp32 accumulators would not
    // fit beside the 16-wave x tile, so each compute item gates its own
    // accumulators, y = q acc in fp32 rounded to bf16 (the same values as
    // gating row-major), in the MFMA layout, with q read from LDS, and
    // stages y: two 32 KiB tiles, so that an item's write-back runs while
    // the next item's MFMAs execute.  Byte b of row r sits at
    //     r PITCH + 16 ((b >> 4) ^ U(r)) + 8 (((b >> 3) & 1) ^ V(r)) + (b & 7),
    //     U(r) = (r & 7) ^ 2 ((r >> 3) & 3),   V(r) = (r >> 3) & 1:
    // the 16 rows of an MFMA tile at one 8-byte channel quad land on 32
    // distinct banks, and a row's 16-byte units stay a permutation of the
    // row's (row-major accesses are conflict-free too).
    auto gaddr = [](int row, int byte) -> int {
        const int u = (row & 7) ^ (((row >> 3) & 3) << 1);
        const int v = (row >> 3) & 1;
        return row * T::PITCH + (((byte >> 4) ^ u) << 4) + ((((byte >> 3) & 1) ^ v) << 3) + (byte & 7);
    };
    // start of the 16-byte unit holding byte b of row r (a 16-byte access
    // there carries the unit's halves swapped where V = 1)
    auto gaddr16 = [](int row, int byte) -> int {
        const int u = (row & 7) ^ (((row >> 3) & 3) << 1);
        return row * T::PITCH + (((byte >> 4) ^ u) << 4);
    };
    // this thread's rows of a row-major 16-byte vector -> tile, and back
    auto put_rows = [&](unsigned char *tile, const u32x4_t *src) {
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int row = i * T::RPL + ld_row;
            const u32x4_t x = src[i];
            const u32x4_t xs2 = ((row >> 3) & 1) ? u32x4_t{x[2], x[3], x[0], x[1]} : x;
            *(u32x4_t *)(&tile[gaddr16(row, ld_seg * 16)]) = xs2;
        }
    };
    auto get_rows = [&](const unsigned char *tile, u32x4_t *dst) {
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int row = i * T::RPL + ld_row;
            const u32x4_t x = *(const u32x4_t *)(&tile[gaddr16(row, ld_seg * 16)]);
            dst[i] = ((row >> 3) & 1) ? u32x4_t{x[2], x[3], x[0], x[1]} : x;
        }
    };
    // y = q acc of compute item j in the MFMA layout (lane: output time
    // 16 nt + n16, channels 4 q4 .. 4 q4 + 3 of this wave's group) -> ys
    auto gate = [&](int j, const f32x4_t *acc) {
        unsigned char *yt = ys + (j & 1) * (kChunk * T::PITCH);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int a = gaddr(16 * nt + n16, (16 * w + 4 * q4) * 2);
            const u32x2_t qv = *(const u32x2_t *)(&qs[a]);
            const u32x2_t yv = {pack_bf16(bf_lo(qv[0]) * acc[nt][0], bf_hi(qv[0]) * acc[nt][1]),
                                pack_bf16(bf_lo(qv[1]) * acc[nt][2], bf_hi(qv[1]) * acc[nt][3])};
            *(u32x2_t *)(&yt[a]) = yv;
        }
    };
    // write-back of compute item j from its ys tile
    auto finish_g = [&](int j) {
        const int c = cp_chunk(j);
        u32x4_t yv[T::NLD];
        get_rows(ys + (j & 1) * (kChunk * T::PITCH), yv);
#pragma unroll
        for (int i = 0; i < T::NLD; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(yv[i], ry, io_off(c, i, true), 0, kFwdStorePolicy);
    };

    // compute item j.  With two staging buffers the previous item's
    // epilogue runs here, while this item's MFMAs execute; its buffer was
    // completed before the last barrier, and the buffer this item stages
    // into was last read before it.  The last item's epilogue follows the
    // walk.  With one buffer, each item's epilogue follows its own barrier.
    auto compute = [&](int j, const frag *Xc) {
        f32x4_t acc[4];
        mma(Xc, acc);
        if constexpr (GSTAGE) {
            if (j > 0) finish_g(j - 1);
            gate(j, acc);
            __syncthreads();
        } else {
            if constexpr (kStBufs == 2) {
                if (j > 0) finish(j - 1);
            }
            stage(j, acc);
            __syncthreads();
            if constexpr (kStBufs == 1) finish(j);
        }
    };

    // ---- the walk: ingest items, each compute item right after its last
    // input chunk.  Xa holds the fragments of every ingest item (registers:
    // each is live only from its ingest to the last compute that reads it,
    // H + 1 items later).  The loop is written once per direction, since
    // which registers hold the oldest input steps of a compute item is fixed
    // at compile time.
    auto walk = [&](auto desc_tag) {
        constexpr bool DESC = decltype(desc_tag)::value;
        frag Xa[NI * M::FPC];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            store_x(kr[i % PF], vr[i % PF]);
            const int n = i + PF;  // the ingest item this slot loads next
            load_kv(n < NI ? (DESC ? S - 1 - n : n - H) : S, n < NI, kr[i % PF], vr[i % PF]);
            if constexpr (GSTAGE) {
                // q of the compute item this ingest completes -> qs, and its
                // slot refilled with the compute item PF ahead
                const int jq = i - H;
                if (jq >= 0) {
                    put_rows(qs, qr[jq % PF][0]);
                    const int nq = jq + PF;
                    load_q(nq < S ? (DESC ? S - 1 - nq : nq) : S, nq < S, qr[jq % PF]);
                }
            }
            __syncthreads();
            read_frags(&Xa[i * M::FPC]);
            const int j = i - H;  // the compute item whose inputs are now all in
            if (j < 0) {
                __syncthreads();  // xs is rewritten by the next ingest
                continue;
            }
            // input step g (in fragments, relative to the span start) of
            // chunk c, oldest first: g = c FPC - NH + kk; its chunk gc and
            // the ingest item that brought gc in
            const int c = DESC ? S - 1 - j : j;
            frag Xc[NX];
#pragma unroll
            for (int kk = 0; kk < NX; ++kk) {
                const int g = c * M::FPC - NH + kk;
                const int gc = g >= 0 ? g / M::FPC : -((-g + M::FPC - 1) / M::FPC);
                const int item = DESC ? S - 1 - gc : gc + H;
                Xc[kk] = Xa[item * M::FPC + (g - gc * M::FPC)];
            }
            compute(j, Xc);
        }
    };
    if constexpr (kWalk == 0) {
        // ---- walk 0.  The span's own chunks first: the first ND need rows
        // from before the span, so their fragments are kept and their outputs
        // deferred.  Then the history rows, while the workgroup of the
        // preceding span reads the same rows as its own last chunks; then the
        // deferred chunks.
        auto ingest = [&](int i, frag *dst) {
            store_x(kr[i % PF], vr[i % PF]);
            const int n = i + PF;
            load_kv(n < NI ? ld_chunk(n) : S, n < NI, kr[i % PF], vr[i % PF]);
            __syncthreads();
            read_frags(dst);
        };
        frag X[NX];
        frag Xsave[ND * M::FPC > 0 ? ND * M::FPC : 1];
#pragma unroll
        for (int c = 0; c < S; ++c) {
            ingest(c, &X[NH]);
            if (c >= ND) {
                compute(c - ND, X);
            } else {
#pragma unroll
                for (int f = 0; f < M::FPC; ++f) Xsave[c * M::FPC + f] = X[NH + f];
                __syncthreads();  // xs is rewritten by the next ingest
            }
#pragma unroll
            for (int i = 0; i < NH; ++i) X[i] = X[i + M::FPC];
        }
        if constexpr (ND > 0) {
            frag Hst[H * M::FPC];
#pragma unroll
            for (int i = S; i < NI; ++i) {
                ingest(i, &Hst[(i - S) * M::FPC]);
                __syncthreads();  // xs is rewritten by the next ingest
            }
            // fragment g (input step relative to the span start) of chunk
            // c's window: history if g < 0 (Hst ends at step -1), else saved
            constexpr int HF = H * M::FPC;
#pragma unroll
            for (int c = 0; c < ND; ++c) {
                if (kStBufs == 1 && c > 0) __syncthreads();  // st is rewritten by this compute
                frag Xc[NX];
#pragma unroll
                for (int kk = 0; kk < NX; ++kk) {
                    const int g = c * M::FPC + kk - NH;
                    Xc[kk] = g < 0 ? Hst[HF + g] : Xsave[g];
                }
                compute(S - ND + c, Xc);
            }
        }
    } else if (desc) {
        walk(std::true_type{});
    } else {
        walk(std::false_type{});
    }
    if constexpr (GSTAGE)
        finish_g(S - 1);
    else if constexpr (kStBufs == 2)
        finish(S - 1);
}

// ---------------------------------------------------------------------------
// Filter gradient, pass 1 (page "04. hardware-aware convolution kernels",
// section 7: block-local partial filter gradients written coalesced, then a
// reduction).  With dz = dy q and x = k v,
//     dh[g, s] = sum_{b, t, d in g} dz[b, t, d] x[b, t - s, d].
// For one 16-channel tile the products dz[t, :] . x[u, :] over the tile's
// channels are a GEMM (rows t of a chunk by rows u of the chunk and its
// history) with the channels as the contraction, so both MFMA operands are
// read row-major: no transpose.  dh[s] sums that product along the diagonal
// t - u = s.  For a 16-row output tile a and input tile b = a - delta, the
// accumulator element (lane n16, q4, i) always has lag 16 delta + 4 q4 + i -
// n16, so every tile pair on one diagonal accumulates into one register tile
// P[delta]; the lags are sorted out once per span.  Each workgroup writes
// its partial dh (one row of l_h floats per 16-channel tile) to ws.
// ---------------------------------------------------------------------------
struct DhParams {
    const void *q, *k, *v, *dy;
    float *ws;          // partial sums: [B * n_spans][D / 16][l_h] (the
                        // direct form: [B * n_spans][D][l_h])
    const void *h;      // filters (the fused forms only)
    void *dq;           // dq output (the fused forms only)
    void *dk, *dv;      // dk, dv outputs (the whole-backward form only)
    int64_t L;
    int32_t D, l_h, n_spans, n_slabs;
    int32_t group_size; // (the fused forms and the direct form)
    int32_t span_rows;  // (the direct form) rows per span
};

// One chunk of q, k, v and dy in flight per workgroup, and at most 128
// VGPRs (4 waves per SIMD): with its 72 KiB of LDS (bf16, l_h = 128) two
// workgroups share a CU and overlap each other's loads, which measured
// faster than two chunks in flight with one workgroup per CU.
template <bool F32, int KH, int S>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void hyena_bwd_dh_kernel(DhParams p) {
    using T = Tr<F32>;
    constexpr int PF = 1;
    constexpr int HROWS = 32 * KH;
    constexpr int H = (HROWS + kChunk - 1) / kChunk;      // history chunks
    constexpr int RING = H + 1;                           // x chunks resident
    constexpr int NDL = 2 * KH + 1;                       // diagonals (16-row units)
    constexpr int PITCH = kSlab * T::EB;
    constexpr int TILE_B = kChunk * PITCH;                // one row-major chunk tile
    constexpr int WALK_B = (RING + 1) * TILE_B;           // x ring + dz tile
    constexpr int LAG_B = kWaves * NDL * 256 * 4;         // every wave's P tiles

    // One LDS area: the x ring and the dz tile during the walk, then the P
    // tiles for the lag sums.
    __shared__ __attribute__((aligned(16))) unsigned char lds[WALK_B > LAG_B ? WALK_B : LAG_B];
    auto xr = [&](int i) -> unsigned char * { return lds + i * TILE_B; };
    unsigned char *const dzs = lds + RING * TILE_B;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int n16 = l & 15;
    const int q4 = l >> 4;

    int bid = blockIdx.x;
    const int slab = bid % p.n_slabs;
    bid /= p.n_slabs;
    const int spn = bid % p.n_spans;
    const int b = bid / p.n_spans;

    const int64_t t_begin = (int64_t)spn * S * kChunk;
    const int64_t t_stop = min(p.L, t_begin + (int64_t)S * kChunk);
    const int64_t base_row = max((int64_t)0, t_begin - HROWS);
    const int c_begin = slab * kSlab;
    const int row_bytes = p.D * T::EB;
    const size_t base_off = ((size_t)b * (size_t)p.L + (size_t)base_row) * (size_t)row_bytes +
                            (size_t)c_begin * T::EB;
    const uint32_t nrec = (uint32_t)((t_stop - base_row) * row_bytes - c_begin * T::EB);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char *)p.q + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char *)p.k + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char *)p.v + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char *)p.dy + base_off, nrec);
    const int row0 = (int)(t_begin - base_row);

    const int ld_row = tid / T::TPR;
    const int ld_seg = tid % T::TPR;
    const bool seg_ok = c_begin + ld_seg * T::VEC < p.D;
    const int ld_base = ld_row * row_bytes + ld_seg * 16;
    auto off = [&](int c, int i, bool need) -> uint32_t {
        const int r = (row0 + c * kChunk + i * T::RPL) * row_bytes + ld_base;
        return (seg_ok && need) ? (uint32_t)r : kOOB;
    };
    // Row-major LDS tiles, 16-byte segment XOR (row & 15): 16 lanes reading
    // the same channels of 16 consecutive rows hit distinct banks.
    auto lds_addr = [&](int row, int byte) -> int {
        return row * PITCH + ((((byte >> 4) ^ (row & 15))) << 4) + (byte & 15);
    };

    u32x4_t kr[PF][T::NLD], vr[PF][T::NLD], qr[PF][T::NLD], dr[PF][T::NLD];
    // chunks -H .. S-1 in order; history chunks need no q, dy
    auto load = [&](int c, int slot) {
        const bool need = c < S;
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const uint32_t o = off(c, i, need);
            const uint32_t og = off(c, i, need && c >= 0);
            kr[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, kLoadPolicy));
            vr[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, kLoadPolicy));
            qr[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, og, 0, kLoadPolicy));
            dr[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rd, og, 0, kLoadPolicy));
        }
    };
    // elementwise product of two 16-byte vectors -> LDS tile (bf16: rounded)
    auto put = [&](unsigned char *tile, const u32x4_t *a, const u32x4_t *b2) {
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int row = i * T::RPL + ld_row;
            u32x4_t xv;
            if constexpr (F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xv[e] = __float_as_uint(__uint_as_float(a[i][e]) * __uint_as_float(b2[i][e]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xv[e] = pack_bf16(bf_lo(a[i][e]) * bf_lo(b2[i][e]), bf_hi(a[i][e]) * bf_hi(b2[i][e]));
            }
            *(u32x4_t *)(&tile[lds_addr(row, ld_seg * 16)]) = xv;
        }
    };

    f32x4_t P[NDL];
#pragma unroll
    for (int d = 0; d < NDL; ++d) P[d] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // this lane's 4 channels of the wave's tile (K of the MFMA)
    const int kbyte = (w * kTile + 4 * q4) * T::EB;

#pragma unroll
    for (int s = 0; s < PF; ++s) load(-H + s, s);
#pragma unroll
    for (int c = -H; c < S; ++c) {
        const int slot = (c + H) % PF;
        unsigned char *xt = xr((c + H) % RING);
        put(xt, kr[slot], vr[slot]);
        if (c >= 0) put(dzs, dr[slot], qr[slot]);
        load(c + PF, slot);
        __syncthreads();
        if (c >= 0) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                // A: dz rows 16a + n16 (as M), channels 4 q4 .. +3 (as K)
                const int ra = 16 * a + n16;
#pragma unroll
                for (int d = 0; d < NDL; ++d) {
                    const int bt = a - d;                         // input tile, may be < 0
                    const int cb = c + (bt < 0 ? -((-bt + 3) / 4) : 0);  // its chunk
                    const int rb = 16 * (bt - 4 * (cb - c)) + n16;       // its row in that chunk
                    const unsigned char *xt2 = xr((cb + H + 4 * RING) % RING);
                    if constexpr (F32) {
                        const f32x4_t av = *(const f32x4_t *)(&dzs[lds_addr(ra, kbyte)]);
                        const f32x4_t bv = *(const f32x4_t *)(&xt2[lds_addr(rb, kbyte)]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            P[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], P[d], 0, 0, 0);
                    } else {
                        typedef short s16x4_t __attribute__((ext_vector_type(4)));
                        const s16x4_t av = *(const s16x4_t *)(&dzs[lds_addr(ra, kbyte)]);
                        const s16x4_t bv = *(const s16x4_t *)(&xt2[lds_addr(rb, kbyte)]);
                        P[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, P[d], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();  // dzs and the oldest x chunk are rewritten next
    }
    // Lags.  Element i of lane (n16, q4) of P[d] is row 4 q4 + i (a dz row)
    // and column n16 (an x row) of a 16 x 16 tile on diagonal d: lag
    // 16 d + 4 q4 + i - n16.  The tiles go to LDS, stored [d][column][row]
    // (the walk's buffers are free after its last barrier), and each lane
    // sums the tile diagonals of its lags in a fixed order: no atomics, and
    // the same bits on every run.
    float *const pt = (float *)lds + w * (NDL * 256);
#pragma unroll
    for (int d = 0; d < NDL; ++d) *(f32x4_t *)(&pt[d * 256 + n16 * 16 + 4 * q4]) = P[d];
    __syncthreads();
    const int tile = slab * kWaves + w;
    if (c_begin + w * kTile < p.D) {
        float *dst = p.ws + ((size_t)(b * p.n_spans + spn) * (size_t)(p.D / kTile) + tile) * p.l_h;
        for (int lag = l; lag < p.l_h; lag += 64) {
            float sum = 0.0f;
            for (int d = 0; d < NDL; ++d) {
                const int m = lag - 16 * d;  // row - column on tile d
                if (m < -15 || m > 15) continue;
                const int c0 = m < 0 ? -m : 0, c1 = m > 0 ? 15 - m : 15;
                for (int col = c0; col <= c1; ++col) sum += pt[d * 256 + col * 17 + m];
            }
            dst[lag] = sum;
        }
    }
}

// ---------------------------------------------------------------------------
// dq and filter-gradient pass 1 in one walk (bf16).  dq = dy (h * x) is the
// forward operator with dy as the gate, and the filter gradient pairs dz =
// dy q with x = k v; both read the same rows of q, k, v and dy, so one pass
// over them serves both (10 bytes per token-channel instead of 8 + 8).  The
// walk is the filter-gradient kernel's (history chunks first, x chunks in an
// LDS ring); the forward's Toeplitz GEMMs (page "04. hardware-aware
// convolution kernels", sections 3-4) read their time-major operand
// fragments from the same ring, keeping the previous chunks' fragments in
// registers.  One swizzle of the ring serves both reads (see lds_addr).
//
// DKV adds dk = v dx and dv = k dx, dx[t] = sum_s h[s] dz[t + s], to the same
// pass, so that q, k, v and dy are read once and dq, dk, dv written once (14
// bytes per token-channel).  That walk runs backwards in time: walk row tau
// is physical row L - 1 - tau, as in the forward kernel's REV form.  Then dx
// is the causal product over dz and completes at each chunk, gated by k and
// v still in registers, while dq runs against the walk.  dz goes to ring A
// and x to a second ring B; the walk runs H chunks past the span (x rows
// only) and completes dq of chunk c - H at chunk c, once x is resident up to
// 32 KH rows past it in walk order.  dq reads the same Toeplitz fragments F,
// with the x fragments taken in reversed row order and the outputs staged in
// reversed row order in a second staging tile (the staged filter taps share
// its memory: they are read before the walk's first barrier, the tile is
// written after it), so the walk keeps two barriers per chunk in 160 KiB of
// LDS.  dq's gate dy is read again then (one tensor; dk and dv late would
// need both k and v again).  The dh products pair x of the chunk with dz
// before it in walk order: the same lag.  dx and its accumulation order are
// those of the forward kernel walked backwards, so dk and dv equal it.
// ---------------------------------------------------------------------------
template <int KH, int S, int PF, bool DKV>
__global__ __launch_bounds__(kThreads) void hyena_bwd_dq_dh_kernel(DhParams p) {
    using T = Tr<false>;
    using M = Mma<false>;
    using frag = M::frag;
    constexpr int HROWS = 32 * KH;
    constexpr int H = (HROWS + kChunk - 1) / kChunk;      // history chunks
    constexpr int RING = H + 1;                           // ring A chunks resident
    constexpr int NZ = DKV ? RING : 1;                    // ring B chunks resident
    constexpr int FH = DKV ? H : 0;                       // chunks walked past the span
    constexpr int NDL = 2 * KH + 1;                       // diagonals (16-row units)
    constexpr int NH = HROWS / M::ROWS;                   // history fragments
    constexpr int NX = NH + M::FPC;                       // fragments one chunk reads
    constexpr int NE = 4 + 2 * KH;                        // Toeplitz fragments
    constexpr int PITCH = T::PITCH;
    constexpr int TILE_B = kChunk * PITCH;
    constexpr int ST_PITCH = kSlab * 4;                   // fp32 staging row, bytes
    constexpr int NST = DKV ? 2 : 1;                      // staging tiles
    constexpr int WALK_B = (RING + NZ) * TILE_B + NST * kChunk * ST_PITCH;  // rings, staging
    constexpr int LAG_B = kWaves * NDL * 256 * 4;
    static_assert(!DKV || kWaves * kHLen * 4 <= kChunk * ST_PITCH, "taps fit the second staging tile");

    __shared__ __attribute__((aligned(16))) unsigned char lds[WALK_B > LAG_B ? WALK_B : LAG_B];
    // chunk c's tiles in ring A (from chunk -H) and ring B (from chunk 0)
    auto xr = [&](int c) -> unsigned char * { return lds + ((c + H + 4 * RING) % RING) * TILE_B; };
    auto zr = [&](int c) -> unsigned char * {
        return lds + (RING + (DKV ? (c + H + 4 * RING) % RING : 0)) * TILE_B;
    };
    unsigned char *const st = lds + (RING + NZ) * TILE_B;
    unsigned char *const st2 = st + (NST - 1) * kChunk * ST_PITCH;  // (DKV) dq staging
    float *hsw;  // this wave's kHLen staged taps
    if constexpr (DKV) {
        hsw = (float *)st2 + (threadIdx.x >> 6) * kHLen;
    } else {
        __shared__ float hs[kWaves][kHLen];
        hsw = hs[threadIdx.x >> 6];
    }

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int n16 = l & 15;
    const int q4 = l >> 4;

    int bid = blockIdx.x;
    const int slab = bid % p.n_slabs;
    bid /= p.n_slabs;
    const int spn = bid % p.n_spans;
    const int b = bid / p.n_spans;

    const int64_t t_begin = (int64_t)spn * S * kChunk;
    const int64_t t_stop = min(p.L, t_begin + (int64_t)S * kChunk);
    const int64_t base_row = max((int64_t)0, t_begin - HROWS);
    const int c_begin = slab * kSlab;
    const int row_bytes = p.D * T::EB;
    // Ring B's tensors are read FH chunks past the span too (the host keeps
    // that window below 2^31 bytes).  DKV: walk row tau is physical row
    // L - 1 - tau, and one window holds walk rows base_row .. t_fut - 1 at
    // physical rows L - t_fut .. L - 1 - base_row for every tensor.
    const int64_t t_fut = min(p.L, t_stop + (int64_t)FH * kChunk);
    const size_t base_off = ((size_t)b * (size_t)p.L + (size_t)(DKV ? p.L - t_fut : base_row)) * (size_t)row_bytes +
                            (size_t)c_begin * T::EB;
    const uint32_t nrec_z = (uint32_t)((t_fut - base_row) * row_bytes - c_begin * T::EB);
    const uint32_t nrec = DKV ? nrec_z : (uint32_t)((t_stop - base_row) * row_bytes - c_begin * T::EB);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char *)p.q + base_off, DKV ? nrec : nrec_z);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char *)p.k + base_off, DKV ? nrec_z : nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char *)p.v + base_off, DKV ? nrec_z : nrec);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char *)p.dy + base_off, DKV ? nrec : nrec_z);
    const __amdgpu_buffer_rsrc_t rdq = make_rsrc((char *)p.dq + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc((char *)(DKV ? p.dk : p.dq) + base_off, nrec);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc((char *)(DKV ? p.dv : p.dq) + base_off, nrec);
    const int row0 = (int)(t_begin - base_row);
    const int rowf = (int)(t_fut - 1 - t_begin);  // (DKV) offset rows of walk row t_begin

    const bool tile_ok = c_begin + w * kTile < p.D;

    const int ld_row = tid / T::TPR;
    const int ld_seg = tid % T::TPR;
    const bool seg_ok = c_begin + ld_seg * T::VEC < p.D;
    const int ld_base = DKV ? ld_seg * 16 - ld_row * row_bytes : ld_row * row_bytes + ld_seg * 16;
    // byte offset of this thread's row i of chunk c (DKV: counted backwards
    // from the window's last row; a walk row past the window's last comes
    // out negative, past every range)
    auto off = [&](int c, int i, bool need) -> uint32_t {
        const int r = DKV ? (rowf - c * kChunk - i * T::RPL) * row_bytes + ld_base
                           : (row0 + c * kChunk + i * T::RPL) * row_bytes + ld_base;
        return (seg_ok && need) ? (uint32_t)r : kOOB;
    };
    // Swizzle of the row-major tiles (LDS of 32 four-byte banks, 128 bytes
    // per cycle): the 16-byte unit XOR U(row) and the 8-byte half XOR V(row),
    //     U = (row & 7) ^ 2 ((row >> 3) & 3),   V = (row >> 3) & 1.
    // 16 consecutive rows at one 8-byte channel quad (the gradient's
    // operands, 16 lanes a cycle) land on 16 distinct 8-byte slots, and 4 row
    // groups of 8 at 16 consecutive channels (the convolution's fragments)
    // on 32 distinct banks.
    auto swz_u = [](int row) -> int { return (row & 7) ^ (((row >> 3) & 3) << 1); };
    auto swz_v = [](int row) -> int { return (row >> 3) & 1; };
    auto lds_addr = [&](int row, int byte) -> int {
        return row * PITCH + ((((byte >> 4) ^ swz_u(row))) << 4) + (((((byte >> 3) & 1) ^ swz_v(row))) << 3) +
               (byte & 7);
    };

    // Ring A (xr) holds the operand of the products that complete at each
    // chunk, ring B (zr) that of the products that complete FH chunks later:
    // x = k v and dz = dy q in time order (dq with dh), dz and x walked
    // backwards (DKV).  The gate of DKV's late product, dy, is read again
    // then: its first read allocates in L2 so that the second mostly hits.
    // (With dk and dv late instead, walking in time order, allocating first
    // reads of k and v took the call from 131 to 100 us for SE and 137 to
    // 116 us for MR; walking backwards, MR takes 112-117 us.)
    const __amdgpu_buffer_rsrc_t rA1 = DKV ? rd : rk, rA2 = DKV ? rq : rv;
    const __amdgpu_buffer_rsrc_t rB1 = DKV ? rk : rd, rB2 = DKV ? rv : rq;
    constexpr int kPolA1 = DKV ? 0 : kLoadPolicy;  // k, or (DKV) dy
    u32x4_t a1r[PF][T::NLD], a2r[PF][T::NLD], b1r[PF][T::NLD], b2r[PF][T::NLD];
    // chunks -H .. S-1+FH in walk order; ring A needs chunks -H .. S-1 and
    // ring B chunks 0 .. S-1+FH
    auto load = [&](int c, int slot) {
        const bool need = c < S;
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const uint32_t o = off(c, i, need);
            const uint32_t og = off(c, i, c >= 0 && c < S + FH);
            a1r[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rA1, o, 0, kPolA1));
            a2r[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rA2, o, 0, kLoadPolicy));
            b2r[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB2, og, 0, kLoadPolicy));
            b1r[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB1, og, 0, kLoadPolicy));
        }
    };
    // elementwise product of two 16-byte vectors, rounded to bf16 -> LDS tile
    // (one 16-byte write per unit, its 8-byte halves swapped where V = 1)
    auto put = [&](unsigned char *tile, const u32x4_t *a, const u32x4_t *b2) {
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int row = i * T::RPL + ld_row;
            u32x4_t xv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xv[e] = pack_bf16(bf_lo(a[i][e]) * bf_lo(b2[i][e]), bf_hi(a[i][e]) * bf_hi(b2[i][e]));
            const u32x4_t wv = swz_v(row) ? u32x4_t{xv[2], xv[3], xv[0], xv[1]} : xv;
            *(u32x4_t *)(&tile[row * PITCH + ((ld_seg ^ swz_u(row)) << 4)]) = wv;
        }
    };
    auto st_addr = [&](int row, int seg) -> int { return row * ST_PITCH + ((seg ^ (row & 15)) << 4); };
    // y = gate * (staged fp32 accumulators) for this thread's rows of chunk
    // c, rounded to bf16 -> out
    auto gate_store = [&](const unsigned char *tile, const u32x4_t *g, const __amdgpu_buffer_rsrc_t &out, int c) {
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int row = i * T::RPL + ld_row;
            const f32x4_t a0 = *(const f32x4_t *)(&tile[st_addr(row, 2 * ld_seg)]);
            const f32x4_t a1 = *(const f32x4_t *)(&tile[st_addr(row, 2 * ld_seg + 1)]);
            u32x4_t yv;
            yv[0] = pack_bf16(bf_lo(g[i][0]) * a0[0], bf_hi(g[i][0]) * a0[1]);
            yv[1] = pack_bf16(bf_lo(g[i][1]) * a0[2], bf_hi(g[i][1]) * a0[3]);
            yv[2] = pack_bf16(bf_lo(g[i][2]) * a1[0], bf_hi(g[i][2]) * a1[1]);
            yv[3] = pack_bf16(bf_lo(g[i][3]) * a1[2], bf_hi(g[i][3]) * a1[3]);
            __builtin_amdgcn_raw_buffer_store_b128(yv, out, off(c, i, true), 0, kStorePolicy);
        }
    };

#pragma unroll
    for (int s = 0; s < PF; ++s) load(-H + s, s);
    // ---- stage this wave's filter (zero outside [0, l_h)), after the first
    // chunks' loads are issued; every tap load unconditional (an index
    // outside the filter reads the row's first tap, then replaced by zero)
    {
        const int g = tile_ok ? (c_begin + w * kTile) / p.group_size : 0;
        const uint16_t *hg = (const uint16_t *)p.h + (size_t)g * p.l_h;
        constexpr int NTL = kHLen / 64;
        uint32_t hv[NTL];
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            const int tap = l + 64 * j - kHOff;
            hv[j] = hg[tile_ok && tap >= 0 && tap < p.l_h ? tap : 0];
        }
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            const int tap = l + 64 * j - kHOff;
            hsw[l + 64 * j] = tile_ok && tap >= 0 && tap < p.l_h ? bf_lo(hv[j]) : 0.0f;
        }
    }
    __syncthreads();  // filters staged

    // Toeplitz operand fragments (B = H^T), as in the forward kernel.
    frag F[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int j = 0; j < 8; ++j) F[e][j] = (__bf16)hsw[16 * e + n16 - 8 * q4 - j + kHOff];
    // Time-major fragment reads (A = X^T: lane n16 = channel 16 w + n16,
    // element j = row 8 q4 + j of a 32-row step): the byte offsets of the
    // eight rows within a tile (the swizzle repeats every 32 rows).
    const int ch = w * kTile + n16;
    int fr_off[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) fr_off[j] = lds_addr(8 * q4 + j, 2 * ch);
    // the same read backwards in time: element j = row 31 - 8 q4 - j
    int fr_rev[DKV ? 8 : 1];
    if constexpr (DKV) {
#pragma unroll
        for (int j = 0; j < 8; ++j) fr_rev[j] = lds_addr(31 - 8 * q4 - j, 2 * ch);
    }
    auto read_frags = [&](const unsigned char *tb, frag *dst) {
#pragma unroll
        for (int kk = 0; kk < M::FPC; ++kk)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                dst[kk][j] = __builtin_bit_cast(__bf16, *(const uint16_t *)(&tb[fr_off[j] + 32 * kk * PITCH]));
    };

    // the previous chunks' fragments in registers (DKV: read from the ring)
    frag X[DKV ? 1 : NX];
    if constexpr (!DKV) {
#pragma unroll
        for (int i = 0; i < NX; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) X[i][j] = (__bf16)0.0f;
    }
    f32x4_t P[NDL];
#pragma unroll
    for (int d = 0; d < NDL; ++d) P[d] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int kbyte = (w * kTile + 4 * q4) * T::EB;  // this lane's 4 channels (gradient K)

    auto chunk_step = [&](const int c) {
        const int slot = (c + H) % PF;
        const bool own = c >= 0 && c < S;  // a span chunk: its own products and the dh products
        const int cg = c - FH;             // the chunk whose late products complete here
        unsigned char *xt = xr(c);
        if (c < S) put(xt, a1r[slot], a2r[slot]);
        // gates of chunk c's own products: dy, or (DKV) k and v
        u32x4_t g1c[T::NLD], g2c[DKV ? T::NLD : 1];
        if (c >= 0) {
            put(zr(c), b1r[slot], b2r[slot]);
            if (own) {
#pragma unroll
                for (int i = 0; i < T::NLD; ++i) g1c[i] = b1r[slot][i];
                if constexpr (DKV) {
#pragma unroll
                    for (int i = 0; i < T::NLD; ++i) g2c[i] = b2r[slot][i];
                }
            }
        }
        // (DKV) dy of chunk cg, dq's gate, read again (L2 hits for the most part)
        u32x4_t dyg[DKV ? T::NLD : 1];
        if constexpr (DKV) {
            if (cg >= 0) {
#pragma unroll
                for (int i = 0; i < T::NLD; ++i)
                    dyg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rd, off(cg, i, true), 0, kLoadPolicy));
            }
        }
        load(c + PF, slot);
        __syncthreads();
        if constexpr (!DKV) {
            if (c < S) read_frags(xt, &X[NH]);
        }
        if (own) {
            const unsigned char *bt_c = zr(c);
            // filter gradient: P[d] += ring B rows (16 a + n16) . ring A rows
            // 16 (a - d) + n16 of this and the previous chunks: dz with x
            // before it in time, or (DKV) x with dz before it in the walk,
            // the same lag either way
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ra = 16 * a + n16;
                typedef short s16x4_t __attribute__((ext_vector_type(4)));
                const s16x4_t av = *(const s16x4_t *)(&bt_c[lds_addr(ra, kbyte)]);
#pragma unroll
                for (int d = 0; d < NDL; ++d) {
                    const int bt = a - d;
                    const int cb = c + (bt < 0 ? -((-bt + 3) / 4) : 0);
                    const int rb = 16 * (bt - 4 * (cb - c)) + n16;
                    const unsigned char *xt2 = xr(cb);
                    const s16x4_t bv = *(const s16x4_t *)(&xt2[lds_addr(rb, kbyte)]);
                    P[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, P[d], 0, 0, 0);
                }
            }
            // the causal product over ring A for chunk c (dq, or (DKV) dx),
            // 16 output rows per tile nt
            if constexpr (DKV) {
                // input step kappa = kk - NH: 32-row block kappa from the
                // chunk's start (chunk c + floor(kappa / 2), half kappa & 1)
                f32x4_t acc[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < NX; ++kk) {
                    const int kap = kk - NH;
                    const unsigned char *xt3 = xr(c + (kap >= 0 ? 0 : -((1 - kap) / 2))) + (kap & 1) * 32 * PITCH;
                    frag xf;
#pragma unroll
                    for (int j = 0; j < 8; ++j) xf[j] = __builtin_bit_cast(__bf16, *(const uint16_t *)(&xt3[fr_off[j]]));
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const int e = nt - 2 * kap;
                        if (e < 0) continue;
                        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, F[e], acc[nt], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) *(f32x4_t *)(&st[st_addr(16 * nt + n16, 4 * w + q4)]) = acc[nt];
            } else {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kk = 0; kk < NX; ++kk) {
                        const int e = nt - 2 * (kk - NH);
                        if (e < 0) continue;
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(X[kk], F[e], acc, 0, 0, 0);
                    }
                    *(f32x4_t *)(&st[st_addr(16 * nt + n16, 4 * w + q4)]) = acc;
                }
            }
        }
        // (DKV) the product over ring B against the walk, dq of chunk cg, ->
        // st2: output tile nt holds rows 63 - 16 nt - n16; input step kappa =
        // kk - NH covers the 32-row block b = 1 - kappa counted from the
        // chunk's start (chunk cg + b / 2, half b % 2), its rows in reverse
        if constexpr (DKV) {
            if (cg >= 0) {
                f32x4_t ga[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) ga[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < NX; ++kk) {
                    const int blk = NH + 1 - kk;
                    const unsigned char *zt = zr(cg + blk / 2) + (blk % 2) * 32 * PITCH;
                    frag zf;
#pragma unroll
                    for (int j = 0; j < 8; ++j) zf[j] = __builtin_bit_cast(__bf16, *(const uint16_t *)(&zt[fr_rev[j]]));
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const int e = nt - 2 * (kk - NH);
                        if (e < 0) continue;
                        ga[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zf, F[e], ga[nt], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) *(f32x4_t *)(&st2[st_addr(63 - 16 * nt - n16, 4 * w + q4)]) = ga[nt];
            }
        }
        __syncthreads();  // st, st2 complete; every read of the oldest ring chunks done
        if (own) {
            if constexpr (DKV) {
                gate_store(st, g2c, rdk, c);  // dk = v dx
                gate_store(st, g1c, rdv, c);  // dv = k dx
            } else {
                gate_store(st, g1c, rdq, c);  // dq = dy (h * x)
            }
        }
        if constexpr (DKV) {
            if (cg >= 0) gate_store(st2, dyg, rdq, cg);  // dq = dy (h * x)
        }
        // the next chunk writes st and st2 only after its first barrier
        if constexpr (!DKV) {
#pragma unroll
            for (int i = 0; i < NH; ++i) X[i] = X[i + M::FPC];
        }
    };
    if constexpr (DKV) {
        // a loop at run time: unrolled, the walk's schedule needs more
        // registers than a wave has
#pragma unroll 1
        for (int c = -H; c < S + FH; ++c) chunk_step(c);
    } else {
#pragma unroll
        for (int c = -H; c < S; ++c) chunk_step(c);
    }
    __syncthreads();  // the staging tile is read; the lag tiles overwrite it
    // Lags, as in the filter-gradient kernel.
    float *const pt = (float *)lds + w * (NDL * 256);
#pragma unroll
    for (int d = 0; d < NDL; ++d) *(f32x4_t *)(&pt[d * 256 + n16 * 16 + 4 * q4]) = P[d];
    __syncthreads();
    const int tile = slab * kWaves + w;
    if (tile_ok) {
        float *dst = p.ws + ((size_t)(b * p.n_spans + spn) * (size_t)(p.D / kTile) + tile) * p.l_h;
        for (int lag = l; lag < p.l_h; lag += 64) {
            float sum = 0.0f;
            for (int d = 0; d < NDL; ++d) {
                const int m = lag - 16 * d;
                if (m < -15 || m > 15) continue;
                const int c0 = m < 0 ? -m : 0, c1 = m > 0 ? 15 - m : 15;
                for (int col = c0; col <= c1; ++col) sum += pt[d * 256 + col * 17 + m];
            }
            dst[lag] = sum;
        }
    }
}

// Pass 2: dh[g, s] = sum over partial rows and over the group's tiles.
// Consecutive threads read consecutive taps of one partial row.
__global__ __launch_bounds__(256) void hyena_bwd_dh_reduce_kernel(const float *ws, float *dh,
                                                                  int rows, int tiles, int tiles_per_group,
                                                                  int l_h, int G) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= G * l_h) return;
    const int g = idx / l_h, s = idx % l_h;
    // term n = r * tiles_per_group + t (partial row r, tile t of the group),
    // added in that order; eight loads in flight before their adds
    const int n_terms = rows * tiles_per_group;
    auto term = [&](int n) -> float {
        const int r = n / tiles_per_group, t = n % tiles_per_group;
        return ws[((size_t)r * tiles + (size_t)g * tiles_per_group + t) * l_h + s];
    };
    float acc = 0.0f;
    int n = 0;
    for (; n + 8 <= n_terms; n += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = term(n + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; n < n_terms; ++n) acc += term(n);
    dh[idx] = acc;
}

typedef void (*KernelFn)(Params);

// Chunks of k, v and q in flight per workgroup: two for both element types.
// In bf16 three (KH = 4: 221 VGPRs against 174) measured 1-2% slower on
// MI355X, at B = 1, L = 8192, D = 4096 and at L = 2^20 alike.
template <bool F32> constexpr int kPrefetch = 2;

// Spans (chunks per workgroup) with a compiled kernel; a requested span is
// rounded down to one of these.  fp32 stops at 4 (register budget).
constexpr int kSpans[] = {1, 2, 4, 8, 16, 32};
constexpr int kNumSpans = sizeof(kSpans) / sizeof(kSpans[0]);
template <bool F32> constexpr int kNumSpansFor = F32 ? 3 : kNumSpans;

// ---------------------------------------------------------------------------
// Chunk-direction forward, for group sizes that are not a multiple of 16
// (down to one filter per channel).  Page "04. hardware-aware convolution
// kernels", section 6: without grouping, the GEMM is formed along the chunk
// direction, since the Toeplitz blocks of one channel's filter are the same
// for every chunk of that channel.  Here, per channel, a 256-row block is
// cut into 16 sub-chunks of 16 rows, and
//     Y[t_out][sub-chunk] = H[t_out][t_in] X[t_in][sub-chunk]
// with t_out the 16 rows of a sub-chunk and t_in the sub-chunk's rows and
// the l_h - 1 rows before it, in steps of 32 rows (the MFMA's K).  The
// Toeplitz operand H is shared by all 16 sub-chunks.
//
// A workgroup (8 waves) owns 64 channels (fp32: 32) and a span of blocks;
// wave w takes channels 8w .. 8w + 7 (fp32: 4w .. 4w + 3).  In LDS every
// channel is a row of times:
//   * x = k v of the block and the 128 rows before it, in a 384-entry ring,
//     so that one 16-byte read is 8 (fp32: 4) consecutive times of the B
//     operand;
//   * q of the block, overwritten in place by y = q acc, so the gate is
//     applied in the MFMA's own layout (lane: 4 consecutive times of one
//     sub-chunk);
//   * the taps as a table of pairs (h[m], h[m-1]) (fp32: single taps), so an
//     A operand register is one 4-byte read; stored in reverse, so the four
//     pairs of one operand lie at rising addresses in operand order.
// Global loads give a thread 4 consecutive rows of 8 (fp32: 4) channels; the
// thread writes them to LDS per channel, 4 times at once, and the epilogue
// reads them back the same way, so every global access is a 16-byte row
// segment.  LDS rows are in 16-byte units XOR-swizzled by the channel's row
// segment, so the 8 segments of a row land in distinct banks.  (A key that
// spread one staging access over all 16 units of a bank cycle measured more
// bank-conflict cycles on gfx950, and no faster.)
// ---------------------------------------------------------------------------
constexpr int kCdBlock = 256;    // rows per block (16 sub-chunks of 16)
constexpr int kCdRing = 384;     // ring entries per channel: a block + 128 history rows
constexpr int kCdTapOff = 32;    // tap tables: entry m + 32 holds tap (pair) m

// Waves per workgroup of the chunk-direction kernel; each wave owns one
// 16-byte row segment of the slab.  Measured at B=1, L=8192, D=4096 on
// MI355X: 8 waves (128-byte row segments, one workgroup per CU) 60 / 67 us
// for SE / MR with one filter per channel; 4 waves (64-byte segments, two
// or three workgroups per CU) 99 / 106 us.
#ifndef HYENA_CD_WAVES
#define HYENA_CD_WAVES 8
#endif
constexpr int kCdWaves = HYENA_CD_WAVES;
constexpr int kCdThreads = 64 * kCdWaves;

template <bool F32> struct CdTr {
    static constexpr int EB = F32 ? 4 : 2;
    static constexpr int VEC = 16 / EB;                  // channels (or times) per 16 bytes
    static constexpr int SLAB = VEC * kCdWaves;          // channels per workgroup (a wave: one row segment)
    static constexpr int SEGS = SLAB / VEC;              // 16-byte segments per row of the slab
    static constexpr int CPW = SLAB / kCdWaves;          // channels per wave
    static constexpr int RING_B = kCdRing * EB;          // LDS bytes per channel ring
    static constexpr int QY_B = kCdBlock * EB;           // LDS bytes per channel gate row
    static_assert(CPW == VEC, "a wave's channels are one row segment (one swizzle key)");
    static_assert(SEGS * (kCdBlock / 4) == kCdThreads, "4 rows x 16 bytes per thread tile a block");
    static_assert(SEGS <= 8, "swizzle keys 0..7");
};

template <bool F32, int KH, bool REV = false, bool DUAL = false>
__global__ __launch_bounds__(kCdThreads) void hyena_fwd_cd_kernel(Params p) {
    using T = CdTr<F32>;
    constexpr int SLAB = T::SLAB;
    constexpr int HROWS = 32 * KH;
    constexpr int PTN = HROWS + 48;      // tap-table entries per channel
    constexpr int NPT = (SLAB * PTN + kCdThreads - 1) / kCdThreads;
    __shared__ __attribute__((aligned(16))) unsigned char xr[SLAB * T::RING_B];
    __shared__ __attribute__((aligned(16))) unsigned char qy[SLAB * T::QY_B];
    // the second gate's rows, overwritten by y2 = g2 acc (two-output form)
    __shared__ __attribute__((aligned(16))) unsigned char qy2[DUAL ? SLAB * T::QY_B : 16];
    __shared__ uint32_t pt[SLAB * PTN];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int n16 = l & 15;
    const int q4 = l >> 4;

    // Work item: workgroups are dealt to the 8 XCDs in turn, each with its
    // own L2; consecutive items (neighbouring slabs, which share 128-byte
    // lines) go to consecutive workgroups of one XCD.
    int bid;
    {
        const int n = gridDim.x, g = blockIdx.x, per = n >> 3, rem = n & 7, x = g & 7;
        bid = x * per + min(x, rem) + (g >> 3);
    }
    const int slab = bid % p.n_slabs;
    bid /= p.n_slabs;
    const int spn = bid % p.n_spans;
    const int b = bid / p.n_spans;

    const int64_t t_begin = (int64_t)spn * p.span_blocks * kCdBlock;
    const int64_t t_stop = min(p.L, t_begin + (int64_t)p.span_blocks * kCdBlock);
    const int nb = (int)((t_stop - t_begin + kCdBlock - 1) / kCdBlock);  // blocks of this span
    const int c_begin = slab * SLAB;
    const int row_bytes = p.D * T::EB;
    const size_t batch_off = (size_t)b * (size_t)p.L * (size_t)row_bytes + (size_t)c_begin * T::EB;
    // Buffer window of `rows` rows of this slab from row r0 (r0 >= 0,
    // rows >= 0): an offset at or past its end reads 0 and drops writes.  An
    // empty window (the history of a span at row 0) has no records at all:
    // its size must not go negative, or the out-of-bounds offset kOOB would
    // land inside it.  Base and size are made wave-uniform explicitly, so the
    // descriptor lives in scalar registers.
    // Under REV the window holds logical rows r0 .. r0 + rows - 1 at
    // physical rows L - r0 - rows .. L - r0 - 1, in decreasing order (see off).
    auto window = [&](const void *base, int64_t r0, int rows) {
        const int n = rows * row_bytes - c_begin * T::EB;
        const int64_t pr0 = REV ? p.L - r0 - (rows > 0 ? rows : 0) : r0;
        const uint64_t a = (uint64_t)((const char *)base + batch_off + (size_t)pr0 * (size_t)row_bytes);
        const uint64_t au = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
        return make_rsrc((const void *)au, (uint32_t)__builtin_amdgcn_readfirstlane(n > 0 ? n : 0));
    };

    // I/O tile of this thread: rows 4 g4 .. 4 g4 + 3 of a block, channels
    // VEC sg .. VEC sg + VEC - 1 (one 16-byte row segment).
    const int sg = tid % T::SEGS;
    const int g4 = tid / T::SEGS;
    const bool seg_ok = c_begin + sg * T::VEC < p.D;
    // byte offset of logical row r of a window of `rows` rows
    auto off = [&](int r, int rows, bool need) -> uint32_t {
        return (seg_ok && need) ? (uint32_t)((REV ? rows - 1 - r : r) * row_bytes + sg * 16) : kOOB;
    };
    // LDS byte address of time index r in channel ch's row (pitch rb)
    auto pos = [&](int ch, int r, int rb) -> int {
        return ch * rb + ((((r / T::VEC) ^ ((ch / T::VEC) & 7))) << 4) + (r % T::VEC) * T::EB;
    };

    constexpr int NG = DUAL ? 2 : 1;  // gates per row
    u32x4_t k0[4], v0[4], q0[NG][4], k1[4], v1[4], q1[NG][4];
    auto load_block = [&](int blk, u32x4_t *kd, u32x4_t *vd, u32x4_t (*qd)[4]) {
        const int64_t r0 = min(t_begin + (int64_t)blk * kCdBlock, t_stop);  // past the span: empty
        const int rows = min(kCdBlock, (int)(t_stop - r0));
        const __amdgpu_buffer_rsrc_t rq = window(p.q, r0, rows);
        const __amdgpu_buffer_rsrc_t rk = window(p.k, r0, rows);
        const __amdgpu_buffer_rsrc_t rv = window(p.v, r0, rows);
        const __amdgpu_buffer_rsrc_t rg = window(DUAL ? p.g2 : p.q, r0, DUAL ? rows : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = off(4 * g4 + i, rows, true);
            kd[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, kLoadPolicy));
            vd[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, kLoadPolicy));
            qd[0][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, kLoadPolicy));
            if constexpr (DUAL)
                qd[1][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rg, o, 0, kLoadPolicy));
        }
    };
    // HBM requests first: the first block, then the history rows before the
    // span (in the first HROWS / 4 row groups), then the taps (L2-resident)
    load_block(0, k0, v0, q0);
    u32x4_t hk[4], hv[4];
    const bool hist = g4 < HROWS / 4;
    if constexpr (HROWS > 0) {
        if (t_begin > 0) {
            // spans start on block boundaries, so every history row of a
            // later span lies at or after row 0
            const int64_t hr0 = t_begin - HROWS;
            const __amdgpu_buffer_rsrc_t rk = window(p.k, hr0, HROWS);
            const __amdgpu_buffer_rsrc_t rv = window(p.v, hr0, HROWS);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t o = off(4 * g4 + i, HROWS, hist);
                hk[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
                hv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
            }
        } else {
            // the first span: the HROWS rows before row 0 are the last rows
            // of the caller's prefix (P rows of kp, vp per batch row; none:
            // zeros), row P + t for time t < 0
            const size_t pre_off = (size_t)b * (size_t)p.P * (size_t)row_bytes + (size_t)c_begin * T::EB;
            const int np = p.P > 0 ? p.P * row_bytes - c_begin * T::EB : 0;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.P > 0 ? (const char *)p.kp + pre_off : (const char *)p.k,
                                                        (uint32_t)(np > 0 ? np : 0));
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.P > 0 ? (const char *)p.vp + pre_off : (const char *)p.v,
                                                        (uint32_t)(np > 0 ? np : 0));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pr = p.P - HROWS + 4 * g4 + i;  // prefix row of time -HROWS + 4 g4 + i
                const uint32_t o = (seg_ok && hist && pr >= 0) ? (uint32_t)(pr * row_bytes + sg * 16) : kOOB;
                hk[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
                hv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
            }
        }
    }
    // Every tap load is issued unconditionally (an index outside the filter
    // reads element 0 and is then replaced by zero), so all of them are in
    // flight together.
    // (one filter per channel, the filter row is the channel: no division)
    uint32_t tap_lo[NPT], tap_hi[NPT];
    auto load_taps = [&](auto gs1_tag) {
        constexpr bool GS1 = decltype(gs1_tag)::value;
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int i = tid + j * kCdThreads;
            const int dl = i / PTN, m = i % PTN - kCdTapOff;
            const int ch = c_begin + dl;
            const bool chok = i < SLAB * PTN && ch < p.D;
            const size_t hrow = chok ? (size_t)(GS1 ? ch : ch / p.group_size) * p.l_h : 0;
            const bool lo_ok = chok && m >= 0 && m < p.l_h;
            const size_t ilo = lo_ok ? hrow + m : 0;
            if constexpr (F32) {
                const uint32_t vlo = ((const uint32_t *)p.h)[ilo];
                tap_lo[j] = lo_ok ? vlo : 0u;
                tap_hi[j] = 0u;
            } else {
                const bool hi_ok = chok && m >= 1 && m <= p.l_h;
                const size_t ihi = hi_ok ? hrow + m - 1 : 0;
                const uint32_t vlo = ((const uint16_t *)p.h)[ilo];
                const uint32_t vhi = ((const uint16_t *)p.h)[ihi];
                tap_lo[j] = lo_ok ? vlo : 0u;
                tap_hi[j] = hi_ok ? vhi : 0u;
            }
        }
    };
    if (p.group_size == 1)
        load_taps(std::true_type{});
    else
        load_taps(std::false_type{});
    // stored reversed (entry e of a channel at PTN - 1 - e), so the entries
    // one MFMA operand takes, e, e - 2, e - 4, e - 6, lie at rising addresses
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const int i = tid + j * kCdThreads;
        if (i < SLAB * PTN) pt[i - i % PTN + PTN - 1 - i % PTN] = tap_lo[j] | (tap_hi[j] << 16);
    }

    // x = k v of rows 4 g4 .. 4 g4 + 3 -> ring index r (a multiple of 4)
    auto put_x = [&](int r, const u32x4_t *kd, const u32x4_t *vd) {
#pragma unroll
        for (int e = 0; e < T::VEC; ++e) {
            const int ch = sg * T::VEC + e;
            if constexpr (F32) {
                u32x4_t xv;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xv[i] = __float_as_uint(__uint_as_float(kd[i][e]) * __uint_as_float(vd[i][e]));
                *(u32x4_t *)(&xr[pos(ch, r, T::RING_B)]) = xv;
            } else {
                const int d = e >> 1;
                float x4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x4[i] = (e & 1) ? bf_hi(kd[i][d]) * bf_hi(vd[i][d]) : bf_lo(kd[i][d]) * bf_lo(vd[i][d]);
                const u32x2_t xv = {pack_bf16(x4[0], x4[1]), pack_bf16(x4[2], x4[3])};
                *(u32x2_t *)(&xr[pos(ch, r, T::RING_B)]) = xv;
            }
        }
    };
    // a gate's rows 4 g4 .. 4 g4 + 3 -> its gate rows (time 4 g4 of the block)
    auto put_q = [&](const u32x4_t *qd, unsigned char *dst) {
#pragma unroll
        for (int e = 0; e < T::VEC; ++e) {
            const int ch = sg * T::VEC + e;
            if constexpr (F32) {
                const u32x4_t qv = {qd[0][e], qd[1][e], qd[2][e], qd[3][e]};
                *(u32x4_t *)(&dst[pos(ch, 4 * g4, T::QY_B)]) = qv;
            } else {
                const int d = e >> 1;
                uint32_t h4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) h4[i] = (e & 1) ? (qd[i][d] >> 16) : (qd[i][d] & 0xffffu);
                const u32x2_t qv = {h4[0] | (h4[1] << 16), h4[2] | (h4[3] << 16)};
                *(u32x2_t *)(&dst[pos(ch, 4 * g4, T::QY_B)]) = qv;
            }
        }
    };
    // ring index of time t (relative to the block start) for a block whose
    // start sits at ring index rb0: (rb0 + t) mod 384, t in [-128, 384)
    auto wrap = [](int r) -> int {
        r = r >= kCdRing ? r - kCdRing : r;
        return r >= kCdRing ? r - kCdRing : r;
    };
    if constexpr (HROWS > 0) {
        if (hist) put_x(128 - HROWS + 4 * g4, hk, hv);  // times -HROWS .. -1 of block 0
    }

    // MFMA lane roles: A = taps (row n16 = output row of a sub-chunk),
    // B = x (column n16 = sub-chunk); the accumulator holds output rows
    // 4 q4 .. 4 q4 + 3 of sub-chunk n16.
    const int lane_t8 = 16 * n16 + 8 * q4;  // B rows of a 32-row step (times)
    const int lane_t4 = 16 * n16 + 4 * q4;  // accumulator rows (fp32: B rows of a group)

    // One block: stage x and q, prefetch the next block, contract, gate,
    // write back.  Blocks alternate between the two register sets.
    // The next block's loads go out before this block is staged (its
    // register set was freed by the previous block), so a block's loads are
    // always in flight.  They are issued unconditionally: past the span the
    // window is empty and they read nothing.  (Behind a branch, the
    // compiler's wait for this block's data would also wait for them.)
    auto process = [&](int blk, const u32x4_t *kd, const u32x4_t *vd, const u32x4_t (*qd)[4],
                       u32x4_t *kn, u32x4_t *vn, u32x4_t (*qn)[4]) {
        const int rb0 = (blk % 3) * 256 + 128 >= kCdRing ? (blk % 3) * 256 + 128 - kCdRing
                                                         : (blk % 3) * 256 + 128;  // (256 blk + 128) mod 384
        load_block(blk + 1, kn, vn, qn);
        put_x(wrap(rb0 + 4 * g4), kd, vd);
        put_q(qd[0], qy);
        if constexpr (DUAL) put_q(qd[1], qy2);
        // B-operand offsets of this lane within a channel's ring row, one per
        // step: the wave's channels share the swizzle key (one row segment),
        // so these serve all of them.  bf16: steps of 32 input rows; the last
        // (ks = KH) covers rows 0 .. 31 of the sub-chunk, of which 16 .. 31
        // have zero taps, so lanes q4 >= 2 then read rows 0 .. 15 again
        // (finite values inside the block) instead of rows past it.  fp32:
        // groups of 16 input rows, lane q4 taking row 4 q4 + s in MFMA s.
        constexpr int NS = F32 ? 2 * KH + 1 : KH + 1;
        int xoff[NS];
#pragma unroll
        for (int ks = 0; ks < NS; ++ks) {
            const int tin0 = -HROWS + (F32 ? 16 : 32) * ks;
            const int lane = F32 ? lane_t4 : (ks == KH ? lane_t8 - ((q4 & 2) << 3) : lane_t8);
            const unsigned r = (unsigned)wrap(rb0 + kCdRing + tin0 + lane);  // in [0, 384)
            xoff[ks] = (int)((((r / T::VEC) ^ (unsigned)(w & 7))) << 4) + (int)(r % T::VEC) * T::EB;
        }
        __syncthreads();
        // The wave's channels are one 16-byte row segment and the host keeps
        // D a whole number of segments, so they lie all inside D or all past
        // it: one wave-uniform test, and no branch between channels (their
        // reads and matrix-core chains overlap).
        const bool wave_in = (int)__builtin_amdgcn_readfirstlane(c_begin + w * T::CPW) < p.D;
#pragma unroll
        for (int cl = 0; cl < T::CPW; ++cl) {
            if (!wave_in) break;
            const int dl = w * T::CPW + cl;
            const unsigned char *xrow = xr + dl * T::RING_B;
            const uint32_t *ptr = pt + dl * PTN;  // reversed tap table of this channel
            f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (F32) {
                f32x4_t xv[NS];
                float tv[NS][4];
#pragma unroll
                for (int gi = 0; gi < NS; ++gi) {
                    xv[gi] = *(const f32x4_t *)(&xrow[xoff[gi]]);
                    const int c = PTN - 1 - (n16 - 4 * q4 - (-HROWS + 16 * gi) + kCdTapOff);  // entry c - s at c + s
#pragma unroll
                    for (int s = 0; s < 4; ++s) tv[gi][s] = __uint_as_float(ptr[c + s]);
                }
#pragma unroll
                for (int gi = 0; gi < NS; ++gi)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[gi][s], xv[gi][s], acc, 0, 0, 0);
            } else {
                u32x4_t xv[NS], hv[NS];
#pragma unroll
                for (int ks = 0; ks < NS; ++ks) {
                    xv[ks] = *(const u32x4_t *)(&xrow[xoff[ks]]);
                    // entries e, e - 2, e - 4, e - 6 of e = n16 - 8 q4 - tin0 + 32
                    const int c = PTN - 1 - (n16 - 8 * q4 - (-HROWS + 32 * ks) + kCdTapOff);
                    hv[ks] = u32x4_t{ptr[c], ptr[c + 2], ptr[c + 4], ptr[c + 6]};
                }
#pragma unroll
                for (int ks = 0; ks < NS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hv[ks]),
                                                                  __builtin_bit_cast(bf16x8_t, xv[ks]), acc, 0, 0, 0);
            }
            // y = q acc in place of q (and y2 = g2 acc in place of g2)
            const int qa = pos(dl, lane_t4, T::QY_B);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                unsigned char *gr = gi == 0 ? qy : qy2;
                if constexpr (F32) {
                    const f32x4_t qv = *(const f32x4_t *)(&gr[qa]);
                    *(f32x4_t *)(&gr[qa]) = qv * acc;
                } else {
                    const u32x2_t qv = *(const u32x2_t *)(&gr[qa]);
                    const u32x2_t yv = {pack_bf16(bf_lo(qv[0]) * acc[0], bf_hi(qv[0]) * acc[1]),
                                        pack_bf16(bf_lo(qv[1]) * acc[2], bf_hi(qv[1]) * acc[3])};
                    *(u32x2_t *)(&gr[qa]) = yv;
                }
            }
        }
        __syncthreads();
        // ---- epilogue: rows 4 g4 .. 4 g4 + 3 back to row-major, 16-byte stores
        const int64_t r0 = t_begin + (int64_t)blk * kCdBlock;
        const int brows = min(kCdBlock, (int)(t_stop - r0));
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const unsigned char *gr = gi == 0 ? qy : qy2;
            u32x4_t yrow[4];
            if constexpr (F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u32x4_t cv = *(const u32x4_t *)(&gr[pos(sg * 4 + e, 4 * g4, T::QY_B)]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) yrow[i][e] = cv[i];
                }
            } else {
                u32x2_t cv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) cv[e] = *(const u32x2_t *)(&gr[pos(sg * 8 + e, 4 * g4, T::QY_B)]);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const u32x2_t a = cv[2 * d], c = cv[2 * d + 1];
                    yrow[0][d] = (a[0] & 0xffffu) | (c[0] << 16);
                    yrow[1][d] = (a[0] >> 16) | (c[0] & 0xffff0000u);
                    yrow[2][d] = (a[1] & 0xffffu) | (c[1] << 16);
                    yrow[3][d] = (a[1] >> 16) | (c[1] & 0xffff0000u);
                }
            }
            const __amdgpu_buffer_rsrc_t ry = window(gi == 0 ? p.y : p.y2, r0, brows);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(yrow[i], ry, off(4 * g4 + i, brows, true), 0, kStorePolicy);
        }
        __syncthreads();  // the gate rows and the oldest ring entries are rewritten next
    };
    for (int blk = 0; blk < nb; blk += 2) {
        process(blk, k0, v0, q0, k1, v1, q1);
        if (blk + 1 >= nb) break;
        process(blk + 1, k1, v1, q1, k0, v0, q0);
    }
}

// ---------------------------------------------------------------------------
// Short filters without the 16-channel grouping (page "04. hardware-aware
// convolution kernels", section 6 gives the chunk-direction GEMM for this
// case; for a few taps the plain sum is cheaper).  With l_h <= 8 taps a
// channel's output needs 8 multiply-adds, far below the fp32 vector ridge, so
// each lane computes the definition directly for 4 channels of one
// row-major segment: x = k v of the last LH rows in registers (fp32, exact
// for bf16 inputs), the channels' taps in registers, y = q * sum_s h[s]
// x[t - s] in fp32, rounded once.  Every access is a coalesced row segment
// (a wave covers 256 consecutive channels) and nothing is transposed, so the
// kernel streams q, k, v and y at the rate of a plain elementwise kernel.
// A wave walks one span of rows after reading the LH - 1 rows before it;
// rows are loaded four at a time, the next four while these are computed.
// Each output's sum runs over s = LH - 1 .. 0 whatever the span, so spans
// give the same bits.
//
// REV walks time backwards (walk row tau is physical row L - 1 - tau), which
// turns the backward's correlation dx[t] = sum_s h[s] dz[t + s] into the same
// causal sum; DUAL gates that sum twice (y = q acc and y2 = g2 acc), as dk =
// v dx and dv = k dx need.  Without REV the rows before row 0 may come from
// a caller prefix (kp, vp: P rows per batch row).
// ---------------------------------------------------------------------------
constexpr int kDirTaps = 8;                // longest filter of the direct kernels
constexpr int kDirCh = 4;                  // channels per lane
constexpr int kDirSlab = 64 * kDirCh;      // channels per wave (one workgroup)
constexpr int kDirBatch = 4;               // rows per load batch

// The direct kernels' shared pieces: the work item, the row window and its
// byte offsets, the segment loads and the taps.
template <bool F32, int LH, bool REV>
struct DirWalk {
    typedef typename std::conditional<F32, u32x4_t, u32x2_t>::type seg_t;
    static constexpr int EB = F32 ? 4 : 2;
    int b, spn, c0, rel0, nrows, nwin, row_bytes;
    bool ok;
    int64_t t0;
    size_t base;  // byte offset of the window's first physical row in a [B, L, D] tensor

    // `tail`: walk rows past the span that the window also holds
    __device__ DirWalk(int64_t L, int D, int n_slabs, int n_spans, int span_rows, int tail = 0) {
        int bid = blockIdx.x;
        const int slab = bid % n_slabs;
        bid /= n_slabs;
        spn = bid % n_spans;
        b = bid / n_spans;
        c0 = slab * kDirSlab + (int)threadIdx.x * kDirCh;
        ok = c0 < D;  // D % 4 == 0: the lane's 4 channels are all in range
        t0 = (int64_t)spn * span_rows;
        const int64_t t1 = min(L, t0 + (int64_t)span_rows);
        const int64_t t2 = min(L, t1 + (int64_t)tail);
        const int64_t r_lo = max((int64_t)0, t0 - (LH - 1));
        row_bytes = D * EB;
        rel0 = (int)(t0 - r_lo);
        nrows = (int)(t1 - t0);
        nwin = (int)(t2 - r_lo);
        // walk rows r_lo .. t2 - 1: physical rows r_lo .. t2 - 1, or (REV)
        // L - t2 .. L - 1 - r_lo in decreasing order (the host keeps the
        // window below 2^31 bytes)
        base = ((size_t)b * (size_t)L + (size_t)(REV ? L - t2 : r_lo)) * (size_t)row_bytes;
    }
    __device__ uint32_t nrec() const { return (uint32_t)(nwin * row_bytes); }
    // byte offset of the lane's segment in walk row t0 + i (i >= -(LH - 1));
    // rows past the span (or, with `past`, past the window): out of range
    __device__ uint32_t off(int i, bool past = false) const {
        const int w = rel0 + i;
        return (ok && (past ? w < nwin : i < nrows)) ? (uint32_t)((REV ? nwin - 1 - w : w) * row_bytes + c0 * EB)
                                                     : kOOB;
    }
    template <int POLICY>
    __device__ static seg_t load(const __amdgpu_buffer_rsrc_t &r, uint32_t o) {
        if constexpr (F32)
            return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, POLICY));
        else
            return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, POLICY));
    }
    __device__ static void store(const seg_t &v, const __amdgpu_buffer_rsrc_t &r, uint32_t o) {
        if constexpr (F32)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, o, 0, kStorePolicy);
        else
            __builtin_amdgcn_raw_buffer_store_b64(v, r, o, 0, kStorePolicy);
    }
    __device__ static float elem(const seg_t &a, int c) {
        if constexpr (F32) return __uint_as_float(a[c]);
        else return (c & 1) ? bf_hi(a[c >> 1]) : bf_lo(a[c >> 1]);
    }
    __device__ static seg_t pack(const float *y) {
        seg_t out;
        if constexpr (F32) {
#pragma unroll
            for (int c = 0; c < kDirCh; ++c) out[c] = __float_as_uint(y[c]);
        } else {
            out[0] = pack_bf16(y[0], y[1]);
            out[1] = pack_bf16(y[2], y[3]);
        }
        return out;
    }
    // taps of the lane's channels (zero past l_h)
    __device__ void taps(const void *h, int group_size, int l_h, float (*hv)[LH]) const {
#pragma unroll
        for (int c = 0; c < kDirCh; ++c) {
            const size_t hrow = ok ? (size_t)((c0 + c) / group_size) * l_h : 0;
#pragma unroll
            for (int s = 0; s < LH; ++s) {
                float t = 0.0f;
                if (ok && s < l_h) t = F32 ? ((const float *)h)[hrow + s] : bf_lo(((const uint16_t *)h)[hrow + s]);
                hv[c][s] = t;
            }
        }
    }
};

template <bool F32, int LH, bool REV, bool DUAL>
__global__ __launch_bounds__(64) void hyena_fwd_direct_kernel(Params p) {
    using W = DirWalk<F32, LH, REV>;
    using seg_t = typename W::seg_t;
    const W wk(p.L, p.D, p.n_slabs, p.n_spans, p.span_rows);
    const uint32_t nrec = wk.nrec();
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char *)p.q + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char *)p.k + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char *)p.v + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc((char *)p.y + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc((const char *)(DUAL ? p.g2 : p.q) + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t ry2 = make_rsrc((char *)(DUAL ? p.y2 : p.y) + wk.base, nrec);

    float hv[kDirCh][LH];
    wk.taps(p.h, p.group_size, p.l_h, hv);
    // xw[s][c] = x of row t - s while row t is computed; before the first
    // row, row -j sits in xw[j - 1] (the first row's shift moves it to xw[j]).
    // History rows (read by the previous span too) use the default,
    // L2-allocating policy; rows before row 0 come from the prefix, if any.
    seg_t kb[2][kDirBatch], vb[2][kDirBatch], qb[2][kDirBatch], gb[2][DUAL ? kDirBatch : 1];
    auto load_batch = [&](int i0, int sl) {
#pragma unroll
        for (int u = 0; u < kDirBatch; ++u) {
            const uint32_t o = wk.off(i0 + u);
            kb[sl][u] = W::template load<kLoadPolicy>(rk, o);
            vb[sl][u] = W::template load<kLoadPolicy>(rv, o);
            qb[sl][u] = W::template load<kLoadPolicy>(rq, o);
            if constexpr (DUAL) gb[sl][u] = W::template load<kLoadPolicy>(rg, o);
        }
    };
    // The history rows' loads are all issued, then the first batch's, before
    // any is used (a row in neither the sequence nor the prefix reads as
    // zero: an offset outside the window); the walk-row selection is uniform
    // per workgroup, so picking the sequence or the prefix is a scalar select.
    const size_t pb = (size_t)wk.b * (size_t)p.P * (size_t)wk.row_bytes;
    const bool has_pre = !REV && p.P > 0;
    const __amdgpu_buffer_rsrc_t rkp =
        make_rsrc(has_pre ? (const char *)p.kp + pb : (const char *)p.k, has_pre ? (uint32_t)(p.P * wk.row_bytes) : 0u);
    const __amdgpu_buffer_rsrc_t rvp =
        make_rsrc(has_pre ? (const char *)p.vp + pb : (const char *)p.v, has_pre ? (uint32_t)(p.P * wk.row_bytes) : 0u);
    seg_t hk[LH > 1 ? LH - 1 : 1], hvv[LH > 1 ? LH - 1 : 1];
#pragma unroll
    for (int j = 1; j < LH; ++j) {
        const bool in_seq = wk.t0 - j >= 0;
        const bool in_pre = !in_seq && has_pre && p.P + wk.t0 - j >= 0;
        const uint32_t o = in_seq ? wk.off(-j)
                           : (in_pre && wk.ok) ? (uint32_t)((p.P + (int)wk.t0 - j) * wk.row_bytes + wk.c0 * W::EB)
                                               : kOOB;
        hk[j - 1] = W::template load<0>(in_seq ? rk : rkp, o);
        hvv[j - 1] = W::template load<0>(in_seq ? rv : rvp, o);
    }
    load_batch(0, 0);
    float xw[LH][kDirCh];
#pragma unroll
    for (int c = 0; c < kDirCh; ++c) xw[LH - 1][c] = 0.0f;
#pragma unroll
    for (int j = 1; j < LH; ++j)
#pragma unroll
        for (int c = 0; c < kDirCh; ++c) xw[j - 1][c] = W::elem(hk[j - 1], c) * W::elem(hvv[j - 1], c);
    for (int i = 0; i < wk.nrows; i += 2 * kDirBatch) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int ib = i + sl * kDirBatch;
            load_batch(ib + kDirBatch, sl ^ 1);
            // the next batch's loads go out before this batch is used: kept
            // in place, so the wait for this batch leaves them in flight
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kDirBatch; ++u) {
#pragma unroll
                for (int s = LH - 1; s > 0; --s)
#pragma unroll
                    for (int c = 0; c < kDirCh; ++c) xw[s][c] = xw[s - 1][c];
                float y1[kDirCh], y2[kDirCh];
#pragma unroll
                for (int c = 0; c < kDirCh; ++c) {
                    xw[0][c] = W::elem(kb[sl][u], c) * W::elem(vb[sl][u], c);
                    float a = 0.0f;
#pragma unroll
                    for (int s = LH - 1; s >= 0; --s) a = __builtin_fmaf(hv[c][s], xw[s][c], a);
                    y1[c] = W::elem(qb[sl][u], c) * a;
                    if constexpr (DUAL) y2[c] = W::elem(gb[sl][u], c) * a;
                }
                W::store(W::pack(y1), ry, wk.off(ib + u));
                if constexpr (DUAL) W::store(W::pack(y2), ry2, wk.off(ib + u));
            }
        }
    }
}

// The whole backward for short filters off the tile, in one walk backwards
// in time (walk row r is physical row L - 1 - r), so that q, k, v and dy are
// read once and dq, dk, dv written once:
//   * dz = dy q and x = k v (fp32) go into register windows of the last LH
//     walk rows, dy into a delay line as long;
//   * dx of row r is the causal sum over the dz window, h[s] dz[r - s] in
//     walk order (= dz[t + s] in time): dk = v dx and dv = k dx, with row r's
//     gates still in registers;
//   * the partial filter gradient pairs row r's x with the dz window:
//     dh[s] gets x[u] dz[u + s] (in time) for each of the span's rows u;
//   * dq needs the LH - 1 rows before it in time, which come after it in the
//     walk: dq of walk row r - (LH - 1) is completed at row r from the x
//     window read backwards, gated by dy from the delay line.
// The walk starts LH - 1 rows before the span (dz only) and runs LH - 1 rows
// past it (x only).  dx and dq sum over the taps in the orders the direct
// forward kernels use, so dk, dv and dq have the same bits as those kernels.
// The partial sums go to ws[B * spans][D][l_h]; a reduction adds them per
// group (pass 2 of page "04. hardware-aware convolution kernels", section 7).
template <bool F32, int LH>
__global__ __launch_bounds__(64) void hyena_bwd_direct_kernel(DhParams p) {
    using W = DirWalk<F32, LH, true>;
    using seg_t = typename W::seg_t;
    const W wk(p.L, p.D, p.n_slabs, p.n_spans, p.span_rows, LH - 1);
    const uint32_t nrec = wk.nrec();
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char *)p.q + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char *)p.k + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char *)p.v + wk.base, nrec);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char *)p.dy + wk.base, nrec);
    // outputs not asked for: an empty window, every store dropped
    const __amdgpu_buffer_rsrc_t rdq = make_rsrc((char *)(p.dq ? p.dq : p.ws) + wk.base, p.dq ? nrec : 0u);
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc((char *)(p.dk ? p.dk : p.ws) + wk.base, p.dk ? nrec : 0u);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc((char *)(p.dv ? p.dv : p.ws) + wk.base, p.dv ? nrec : 0u);

    float hv[kDirCh][LH];
    wk.taps(p.h, p.group_size, p.l_h, hv);
    // windows: zw[s] = dz of walk row r - s, xw[s] = x of row r - s, yw[s]
    // = dy of row r - s; rows outside the walk are zero
    float zw[LH][kDirCh], xw[LH][kDirCh], yw[LH][kDirCh], P[kDirCh][LH];
#pragma unroll
    for (int s = 0; s < LH; ++s)
#pragma unroll
        for (int c = 0; c < kDirCh; ++c) zw[s][c] = xw[s][c] = yw[s][c] = P[c][s] = 0.0f;
    // walk rows i = -(LH - 1) .. nrows + LH - 2 relative to the span start:
    // dz where i < nrows, x where i >= 0 (both zero past the sequence)
    const int i_begin = -(LH - 1), i_end = wk.nrows + LH - 1;
    seg_t kb[2][kDirBatch], vb[2][kDirBatch], qb[2][kDirBatch], db[2][kDirBatch];
    auto load_batch = [&](int i0, int sl) {
#pragma unroll
        for (int u = 0; u < kDirBatch; ++u) {
            const int i = i0 + u;
            const bool in_walk = i < i_end && (int)wk.t0 + i >= 0;
            const uint32_t oz = (in_walk && i < wk.nrows) ? wk.off(i) : kOOB;
            const uint32_t ox = (in_walk && i >= 0) ? wk.off(i, true) : kOOB;
            qb[sl][u] = W::template load<kLoadPolicy>(rq, oz);
            db[sl][u] = W::template load<kLoadPolicy>(rd, oz);
            kb[sl][u] = W::template load<kLoadPolicy>(rk, ox);
            vb[sl][u] = W::template load<kLoadPolicy>(rv, ox);
        }
    };
    load_batch(i_begin, 0);
    for (int i = i_begin; i < i_end; i += 2 * kDirBatch) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int ib = i + sl * kDirBatch;
            load_batch(ib + kDirBatch, sl ^ 1);
            // the next batch's loads go out before this batch is used
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kDirBatch; ++u) {
                const int r = ib + u;
#pragma unroll
                for (int s = LH - 1; s > 0; --s)
#pragma unroll
                    for (int c = 0; c < kDirCh; ++c) {
                        zw[s][c] = zw[s - 1][c];
                        xw[s][c] = xw[s - 1][c];
                        yw[s][c] = yw[s - 1][c];
                    }
                float yk[kDirCh], yv[kDirCh], yq[kDirCh];
#pragma unroll
                for (int c = 0; c < kDirCh; ++c) {
                    const float kx = W::elem(kb[sl][u], c), vx = W::elem(vb[sl][u], c);
                    const float dyv = W::elem(db[sl][u], c);
                    zw[0][c] = dyv * W::elem(qb[sl][u], c);
                    xw[0][c] = kx * vx;
                    yw[0][c] = dyv;
                    // dx of row r (zero outside the span: its stores drop)
                    float a = 0.0f;
#pragma unroll
                    for (int s = LH - 1; s >= 0; --s) a = __builtin_fmaf(hv[c][s], zw[s][c], a);
                    yk[c] = vx * a;
                    yv[c] = kx * a;
                    // partial dh: x of row r (zero outside the span's rows
                    // and the tail) with dz of the rows after it in time
                    if (r >= 0 && r < wk.nrows) {
#pragma unroll
                        for (int s = 0; s < LH; ++s) P[c][s] = __builtin_fmaf(xw[0][c], zw[s][c], P[c][s]);
                    }
                    // dq of walk row r - (LH - 1): x of the rows before it in time
                    float aq = 0.0f;
#pragma unroll
                    for (int s = LH - 1; s >= 0; --s) aq = __builtin_fmaf(hv[c][s], xw[LH - 1 - s][c], aq);
                    yq[c] = yw[LH - 1][c] * aq;
                }
                if (r >= 0 && r < wk.nrows) {
                    W::store(W::pack(yk), rdk, wk.off(r));
                    W::store(W::pack(yv), rdv, wk.off(r));
                }
                const int rq_row = r - (LH - 1);
                if (rq_row >= 0 && rq_row < wk.nrows) W::store(W::pack(yq), rdq, wk.off(rq_row));
            }
        }
    }
    if (wk.ok) {
        float *dst = p.ws + ((size_t)(wk.b * p.n_spans + wk.spn) * (size_t)p.D + (size_t)wk.c0) * p.l_h;
#pragma unroll
        for (int c = 0; c < kDirCh; ++c)
#pragma unroll
            for (int s = 0; s < LH; ++s)
                if (s < p.l_h) dst[c * p.l_h + s] = P[c][s];
    }
}

// dh of an empty problem (no rows): zeros, written by a kernel so that a
// call captured into a graph records kernels only.
__global__ __launch_bounds__(256) void hyena_zero_kernel(float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = 0.0f;
}

// Pass 2 for the direct backward: dh[g, s] = sum over the partial rows and
// the group's channels of ws[row][channel][s], rows outer, channels inner.
__global__ __launch_bounds__(256) void hyena_bwd_direct_dh_reduce_kernel(const float *ws, float *dh, int rows,
                                                                         int D, int group_size, int l_h, int G) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= G * l_h) return;
    const int g = idx / l_h, s = idx % l_h;
    // term n = r * group_size + c, added in that order; eight loads in
    // flight before their adds
    const int n_terms = rows * group_size;
    auto term = [&](int n) -> float {
        const int r = n / group_size, c = n % group_size;
        return ws[((size_t)r * D + (size_t)g * group_size + c) * l_h + s];
    };
    float acc = 0.0f;
    int n = 0;
    for (; n + 8 <= n_terms; n += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = term(n + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += t[u];
    }
    for (; n < n_terms; ++n) acc += term(n);
    dh[idx] = acc;
}

// ---------------------------------------------------------------------------
// Filter gradient, pass 1, for group sizes off the 16-channel tile and
// filters of more than 8 taps (page "04. hardware-aware convolution
// kernels", section 7: block-local partial filter gradients, then a
// reduction).  Per channel d and tap s < l_h,
//     ws[b * n_spans + span][d][s] = sum_{t in span} dz[b, t, d] x[b, t - s, d],
// with dz = dy q and x = k v formed in fp32 (exact for bf16 inputs); the
// reduction adds the rows and the group's channels.  Without a shared
// filter there is no channel dimension to contract on the matrix cores, so
// the lag products are fp32 multiply-adds.
//
// A workgroup owns kLagCh channels of one batch row and a span of rows,
// walked in 64-row blocks.  dz of the block and x of the block and the 128
// rows before it sit in LDS, time-major, so the 64 lanes of a wave (one
// channel each) read 64 consecutive words.  Wave w takes tap group
// jg = w % NG2 (taps 16 jg .. 16 jg + 15) and time slice jt = w / NG2 of
// every block (64 NG2 / 8 rows), in steps of 8 rows: 8 values of dz and a
// window of 23 values of x, then 128 multiply-adds from registers.  Each
// block's products are summed on their own and then added to the span's, and
// the time slices are added in a fixed order at the end, so the result is the
// same run to run.  The next block's rows are loaded while this one is
// summed.
// ---------------------------------------------------------------------------
constexpr int kLagCh = 64;        // channels per workgroup
constexpr int kLagRing = 256;     // x rows per channel in LDS (a block, the 128 before it, slack)
constexpr int kLagSpanRows = 1024;

template <bool F32, int NG2>
__global__ __launch_bounds__(512) void hyena_bwd_dh_lag_kernel(DhParams p) {
    constexpr int EB = F32 ? 4 : 2;
    constexpr int REPS = 8 / NG2;   // time slices of a block
    constexpr int RPT = 64 / REPS;  // rows per slice
    constexpr int NT = 16 * NG2;    // taps this workgroup sums (>= l_h)
    constexpr int NLD = F32 ? 2 : 1;  // 16-byte loads per tensor per thread and block
    __shared__ float xs[kLagRing][kLagCh];
    __shared__ float zs[64][kLagCh];

    const int tid = threadIdx.x, w = tid >> 6, cl = tid & 63;
    const int jg = w % NG2, jt = w / NG2;
    int bid = blockIdx.x;
    const int slab = bid % p.n_slabs;
    bid /= p.n_slabs;
    const int spn = bid % p.n_spans;
    const int b = bid / p.n_spans;
    const int64_t t_begin = (int64_t)spn * p.span_rows;
    const int64_t t_stop = min(p.L, t_begin + (int64_t)p.span_rows);
    const int nblk = (int)((t_stop - t_begin + 63) / 64);
    const int c_begin = slab * kLagCh;
    const int row_bytes = p.D * EB;
    const size_t batch_off = (size_t)b * (size_t)p.L * (size_t)row_bytes + (size_t)c_begin * EB;

    // loader role: row lr of a 64-row block, 8 channels from 8 sg (bf16: one
    // 16-byte access; fp32: two)
    const int lr = tid >> 3, sg = tid & 7;
    auto window = [&](const void *base, int64_t r0, int rows) {
        const int n = rows * row_bytes - c_begin * EB;
        return make_rsrc((const char *)base + batch_off + (size_t)r0 * (size_t)row_bytes, (uint32_t)(n > 0 ? n : 0));
    };
    // byte offset of window row r, this thread's channels (half h), or
    // outside every window (fp32: each half is 4 channels)
    auto off = [&](int r, int h) -> uint32_t {
        const bool ok = r >= 0 && c_begin + sg * 8 + 4 * h < p.D;
        return ok ? (uint32_t)(r * row_bytes + sg * 8 * EB + 16 * h) : kOOB;
    };
    // 8 fp32 values of a * b for this thread's row segment
    auto prod8 = [&](const u32x4_t *a, const u32x4_t *c, float *out) {
        if constexpr (F32) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) out[4 * h + e] = __uint_as_float(a[h][e]) * __uint_as_float(c[h][e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[2 * e] = bf_lo(a[0][e]) * bf_lo(c[0][e]);
                out[2 * e + 1] = bf_hi(a[0][e]) * bf_hi(c[0][e]);
            }
        }
    };
    // ring row of time t (t >= t_begin - 128)
    auto ring = [&](int64_t t) -> int { return (int)((t - t_begin + 128) & (kLagRing - 1)); };

    // the 128 rows of x before the span (rows before 0 read as zero)
    {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t r0 = t_begin - 128 + 64 * half;
            const int64_t c0 = max(r0, (int64_t)0);
            const int rows = (int)(r0 + 64 - c0);  // rows of this block at or after row 0
            const __amdgpu_buffer_rsrc_t rk = window(p.k, c0, rows);
            const __amdgpu_buffer_rsrc_t rv = window(p.v, c0, rows);
            const int rel = (int)(r0 - c0);  // <= 0
            u32x4_t kk[NLD], vv[NLD];
#pragma unroll
            for (int h = 0; h < NLD; ++h) {
                const uint32_t o = off(lr + rel, h);
                kk[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
                vv[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
            }
            float x8[8];
            prod8(kk, vv, x8);
            const int rr = ring(r0 + lr);
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[rr][sg * 8 + e] = x8[e];
        }
    }
    // one block's rows of dy, q, k, v in registers
    u32x4_t dy_r[NLD], q_r[NLD], k_r[NLD], v_r[NLD];
    auto load_blk = [&](int blk) {
        const int64_t r0 = min(t_begin + 64 * (int64_t)blk, t_stop);
        const int rows = (int)min((int64_t)64, t_stop - r0);
        const __amdgpu_buffer_rsrc_t rd = window(p.dy, r0, rows), rq = window(p.q, r0, rows),
                                     rk = window(p.k, r0, rows), rv = window(p.v, r0, rows);
#pragma unroll
        for (int h = 0; h < NLD; ++h) {
            const uint32_t o = off(lr, h);
            dy_r[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rd, o, 0, kLoadPolicy));
            q_r[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, kLoadPolicy));
            k_r[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
            v_r[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
        }
    };
    load_blk(0);

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    for (int blk = 0; blk < nblk; ++blk) {
        const int64_t t0 = t_begin + 64 * (int64_t)blk;
        {
            float z8[8], x8[8];
            prod8(dy_r, q_r, z8);
            prod8(k_r, v_r, x8);
            const int rr = ring(t0 + lr);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                zs[lr][sg * 8 + e] = z8[e];
                xs[rr][sg * 8 + e] = x8[e];
            }
        }
        load_blk(blk + 1);  // past the span: an empty window, nothing read
        __syncthreads();
        float bacc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) bacc[i] = 0.0f;
#pragma unroll
        for (int m = 0; m < RPT / 8; ++m) {
            const int u0 = jt * RPT + 8 * m;  // first row of this step, relative to t0
            float z8[8], xw[23];
#pragma unroll
            for (int u = 0; u < 8; ++u) z8[u] = zs[u0 + u][cl];
            // xw[i] = x[t0 + u0 - 16 jg - 15 + i]
#pragma unroll
            for (int i = 0; i < 23; ++i) xw[i] = xs[ring(t0 + u0 - 16 * jg - 15 + i)][cl];
            // row u, tap 16 jg + k: x index u - k + 15
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int k = 0; k < 16; ++k) bacc[k] = fmaf(z8[u], xw[u - k + 15], bacc[k]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += bacc[i];
        __syncthreads();  // zs and the oldest ring rows are rewritten next
    }
    // the time slices' sums, added in slice order; red[jt][cl][tap] in xs
    float *red = &xs[0][0];
    constexpr int RP = NT + 1;  // row pitch (words) of one channel's taps
    static_assert(REPS * kLagCh * RP <= kLagRing * kLagCh, "reduction fits the ring");
#pragma unroll
    for (int k = 0; k < 16; ++k) red[(jt * kLagCh + cl) * RP + 16 * jg + k] = acc[k];
    __syncthreads();
    float *ws = p.ws + ((size_t)(b * p.n_spans + spn) * p.D + c_begin) * p.l_h;
    for (int o = tid; o < kLagCh * NT; o += 512) {
        const int c = o / NT, sidx = o % NT;
        if (c_begin + c >= p.D || sidx >= p.l_h) continue;
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < REPS; ++r) sum += red[(r * kLagCh + c) * RP + sidx];
        ws[(size_t)c * p.l_h + sidx] = sum;
    }
}

// ---------------------------------------------------------------------------
// The same partial filter gradients in bf16 on the matrix cores.  For one
// channel, with dz = dy q and x = k v each rounded once to bf16 (the
// grouped kernels' dh operands), take an input step of 32 rows from t0 and
//     D[i][j] = sum_{k<32} x[t0 - 8 i + k] * dz[t0 + j + k],
// the product of A[i][k] = x[t0 - 8 i + k] (16 x 32) and B[k][j] =
// dz[t0 + j + k] (32 x 16), i.e. v_mfma_f32_16x16x32_bf16.  Every term of
// D[i][j] pairs dz at time t with x at t - s for the one lag s = 8 i + j, so
// the columns j < 8 give each lag s < 128 once (the columns j >= 8 are not
// used), and steps t0 = S0 - 32, S0, ..., 32 apart, with dz zero outside the
// span's rows [S0, S1), sum every term of the span exactly once.  One MFMA
// per channel and 32 rows replaces 32 * 128 fp32 multiply-adds, and each
// accumulator element already holds one lag: no diagonal sums.
//
// A workgroup owns kLagCh channels and a span (as the fp32 kernel), walked
// in 128-row blocks; wave w takes channels 8 w .. 8 w + 7.  In LDS each
// channel has a time ring of x (512 rows, 16-byte aligned runs of 8 times,
// so an A operand is one 16-byte read) and two rings of dz as dword pairs,
// (dz[2m], dz[2m+1]) and (dz[2m+1], dz[2m+2]), so that a B operand, which
// starts at any time, is four dwords of one of them; four dwords past each
// dz ring's end repeat its first four, so those four never wrap.  Rings are
// rotated by 16 bytes per channel segment (channel / 8) so that one staging
// write of a wave (8 segments x 8 row pairs) covers the banks evenly.  A
// thread loads two consecutive rows of one 16-byte channel segment; the
// next block's rows are loaded while this block's steps run.
// ---------------------------------------------------------------------------
constexpr int kLmBlock = 128;       // rows per block
constexpr int kLmXRing = 512;       // x ring, times per channel
constexpr int kLmZDw = 128;         // dz ring, dwords per copy (256 times)
// the second dz copy starts 144 dwords (16 banks) after the first, so the
// two copies' dwords that one 16-lane group of a B read takes use disjoint banks
constexpr int kLmZCopy = kLmZDw + 16;
constexpr int kLmZPitch = 2 * kLmZCopy;  // dz dwords per channel (two copies, each with 4 repeated)

__global__ __launch_bounds__(512) void hyena_bwd_dh_lag_mfma_kernel(DhParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t xr[kLagCh * kLmXRing];
    __shared__ __attribute__((aligned(16))) uint32_t zr[kLagCh * kLmZPitch];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int n16 = l & 15, q4 = l >> 4;
    int bid = blockIdx.x;
    const int slab = bid % p.n_slabs;
    bid /= p.n_slabs;
    const int spn = bid % p.n_spans;
    const int b = bid / p.n_spans;
    const int64_t S0 = (int64_t)spn * p.span_rows;
    const int64_t S1 = min(p.L, S0 + (int64_t)p.span_rows);
    const int nblk = (int)((S1 - S0 + kLmBlock - 1) / kLmBlock);
    const int c_begin = slab * kLagCh;
    const int row_bytes = p.D * 2;
    const size_t batch_off = (size_t)b * (size_t)p.L * (size_t)row_bytes + (size_t)c_begin * 2;

    // loader role: rows 2 rg, 2 rg + 1 of a block, channels 8 sg .. 8 sg + 7
    const int sg = tid & 7, rg = tid >> 3;
    const bool seg_ok = c_begin + sg * 8 < p.D;
    // rows [r_lo, r_hi) of a tensor (0 <= r_lo <= r_hi <= L): this thread's
    // rows r0 + 2 rg and r0 + 2 rg + 1, zero outside the window
    auto load2 = [&](const void *base, int64_t r0, int64_t r_lo, int64_t r_hi, u32x4_t *dst, auto pol_tag) {
        constexpr int pol = decltype(pol_tag)::value;
        const int n = (int)(r_hi - r_lo) * row_bytes - c_begin * 2;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((const char *)base + batch_off + (size_t)r_lo * (size_t)row_bytes, (uint32_t)(n > 0 ? n : 0));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t r = r0 + 2 * rg + u;
            const uint32_t o = (seg_ok && r >= r_lo && r < r_hi) ? (uint32_t)((r - r_lo) * row_bytes + sg * 16) : kOOB;
            dst[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, pol));
        }
    };
    const std::integral_constant<int, 0> kAlloc;              // L2-allocating loads
    const std::integral_constant<int, kLoadPolicy> kStream;   // streaming loads
    // bf16 (round to nearest even) of the fp32 product of channel e of a, c
    auto prod = [](const u32x4_t &a, const u32x4_t &c, int e) -> uint32_t {
        const float f = (e & 1) ? bf_hi(a[e >> 1]) * bf_hi(c[e >> 1]) : bf_lo(a[e >> 1]) * bf_lo(c[e >> 1]);
        return pack_bf16(f, 0.0f) & 0xffffu;
    };
    // x of times t, t + 1 (t even) for this thread's 8 channels -> x ring
    auto put_x = [&](int64_t t, const u32x4_t *kk, const u32x4_t *vv) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = sg * 8 + e;
            const uint32_t d = prod(kk[0], vv[0], e) | (prod(kk[1], vv[1], e) << 16);
            const int pe = (int)((t + 8 * sg) & (kLmXRing - 1));
            *(uint32_t *)(&xr[ch * kLmXRing + pe]) = d;
        }
    };
    // dz of times t, t + 1 (t even) -> both dz rings (and their repeats)
    auto put_z = [&](int64_t t, const u32x4_t *dd, const u32x4_t *qq) {
        const int m = (int)(t >> 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = sg * 8 + e;
            const uint32_t z0 = prod(dd[0], qq[0], e), z1 = prod(dd[1], qq[1], e);
            uint32_t *z = zr + ch * kLmZPitch;
            const int p0 = (m + 4 * sg) & (kLmZDw - 1);        // copy 0: (dz[t], dz[t+1])
            z[p0] = z0 | (z1 << 16);
            if (p0 < 4) z[kLmZDw + p0] = z0 | (z1 << 16);
            uint16_t *z1h = (uint16_t *)(z + kLmZCopy);         // copy 1: (dz[2m'+1], dz[2m'+2])
            const int ph = (m - 1 + 4 * sg) & (kLmZDw - 1);      // dz[t]: upper half of pair t/2 - 1
            const int pl = (m + 4 * sg) & (kLmZDw - 1);          // dz[t+1]: lower half of pair t/2
            z1h[2 * ph + 1] = (uint16_t)z0;
            if (ph < 4) z1h[2 * (kLmZDw + ph) + 1] = (uint16_t)z0;
            z1h[2 * pl] = (uint16_t)z1;
            if (pl < 4) z1h[2 * (kLmZDw + pl)] = (uint16_t)z1;
        }
    };

    // dz rings start at zero (times before the span read as zero); the 160
    // rows of x before the span (zero before row 0)
    // every load of the history rows and of the first block is issued
    // before any is used (the second history pass: 32 rows, threads rg < 16)
    u32x4_t kk[2], vv[2], kk2[2], vv2[2];
    const int64_t hlo = max((int64_t)0, S0 - 160);
    load2(p.k, S0 - 128, hlo, S0, kk, kAlloc);
    load2(p.v, S0 - 128, hlo, S0, vv, kAlloc);
    const int64_t h2 = rg < 16 ? S0 - 160 : S0;  // threads rg >= 16: rows at S0 and past, outside the window
    load2(p.k, h2, hlo, S0, kk2, kAlloc);
    load2(p.v, h2, hlo, S0, vv2, kAlloc);
    u32x4_t dy_r[2], q_r[2], k_r[2], v_r[2];
    auto load_blk = [&](int blk) {
        const int64_t r0 = S0 + (int64_t)blk * kLmBlock;
        load2(p.dy, r0, S0, S1, dy_r, kStream);
        load2(p.q, r0, S0, S1, q_r, kStream);
        // k and v allocate in L2: the next span reads its last rows as history
        load2(p.k, r0, S0, S1, k_r, kAlloc);
        load2(p.v, r0, S0, S1, v_r, kAlloc);
    };
    load_blk(0);
    for (int i = tid; i < kLagCh * kLmZPitch; i += 512) zr[i] = 0u;
    put_x(S0 - 128 + 2 * rg, kk, vv);
    if (rg < 16) put_x(S0 - 160 + 2 * rg, kk2, vv2);
    __syncthreads();  // the dz rings are zero before any block writes them

    // the wave's channels lie all inside D or all past it (D is a whole
    // number of 8-channel segments)
    const int ch0 = w * 8;
    const bool wave_in = (int)__builtin_amdgcn_readfirstlane(c_begin + ch0) < p.D;
    f32x4_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int rot = 8 * (ch0 >> 3);  // the wave's channels share one segment (rotation)
    for (int blk = 0; blk <= nblk; ++blk) {
        const int64_t bs = S0 + (int64_t)blk * kLmBlock;
        // this block's rows (past the span, or the block after the last: zeros)
        put_x(bs + 2 * rg, k_r, v_r);
        put_z(bs + 2 * rg, dy_r, q_r);
        if (blk < nblk) load_blk(blk + 1);  // the block after the last: an empty window
        __syncthreads();
        const int nk = blk < nblk ? kLmBlock / 32 : 1;
        if (wave_in) {
            for (int ks = 0; ks < nk; ++ks) {
                const int64_t t0 = bs - 32 + 32 * ks;
                // A: x[t0 - 8 n16 + 8 q4 .. + 7]; B: dz[t0 + n16 + 8 q4 .. + 7]
                const int pa = (int)((t0 - 8 * n16 + 8 * q4 + rot) & (kLmXRing - 1));
                const int64_t e0 = t0 + n16 + 8 * q4;
                const int par = (int)(e0 & 1);
                const int pb = par * kLmZCopy + (int)(((e0 - par) / 2 + 4 * (ch0 >> 3)) & (kLmZDw - 1));
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const u32x4_t av = *(const u32x4_t *)(&xr[(ch0 + c) * kLmXRing + pa]);
                    const uint32_t *zb = zr + (ch0 + c) * kLmZPitch + pb;
                    const u32x4_t bv = {zb[0], zb[1], zb[2], zb[3]};
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                     __builtin_bit_cast(bf16x8_t, bv), acc[c], 0, 0, 0);
                }
            }
        }
        __syncthreads();  // the rings' oldest entries are rewritten next
    }
    // lane (n16, q4), element r: lag 8 (4 q4 + r) + n16 (columns n16 < 8)
    if (wave_in && n16 < 8) {
        float *ws = p.ws + ((size_t)(b * p.n_spans + spn) * p.D + c_begin + ch0) * p.l_h;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 8 * (4 * q4 + r) + n16;
                if (s < p.l_h) ws[(size_t)c * p.l_h + s] = acc[c][r];
            }
    }
}

// Kernel families and their compiled span counts (indices into kSpans).
enum Family { kFwd = 0, kRevDual = 1, kDh = 2, kCd = 3, kDqDh = 4, kBwd = 5, kCdRevDual = 6 };
// (the chunk-direction kernel takes its span at run time: one entry)
template <bool F32, int Fam> constexpr int kSpanCount =
    Fam == kFwd ? kNumSpansFor<F32> : Fam == kRevDual ? (F32 ? 2 : 4) : Fam == kDh ? (F32 ? 3 : 5)
    : Fam == kDqDh || Fam == kBwd ? 5 : 1;

typedef void (*DhFn)(DhParams);
template <bool F32, int Fam> struct FnType { typedef KernelFn type; };
template <bool F32> struct FnType<F32, kDh> { typedef DhFn type; };
template <bool F32> struct FnType<F32, kDqDh> { typedef DhFn type; };
template <bool F32> struct FnType<F32, kBwd> { typedef DhFn type; };

template <bool F32, int Fam, int KH, int Sp>
constexpr typename FnType<F32, Fam>::type kernel_of() {
    if constexpr (Fam == kFwd)
        return hyena_fwd_kernel<F32, KH, kPrefetch<F32>, Sp, false, false>;
    else if constexpr (Fam == kRevDual)
        return hyena_fwd_kernel<F32, KH, kPrefetch<F32>, Sp, true, true>;
    else if constexpr (Fam == kDh)
        return hyena_bwd_dh_kernel<F32, KH, Sp>;
    else if constexpr (Fam == kDqDh)
        return hyena_bwd_dq_dh_kernel<KH, Sp, 1, false>;  // bf16 only
    else if constexpr (Fam == kBwd)
        return hyena_bwd_dq_dh_kernel<KH, Sp, 1, true>;  // bf16 only
    else if constexpr (Fam == kCdRevDual)
        return hyena_fwd_cd_kernel<F32, KH, true, true>;
    else
        return hyena_fwd_cd_kernel<F32, KH>;
}

// The bf16 forward with 16 waves: 256-channel slabs, so every row segment a
// workgroup reads or writes is 512 contiguous bytes.  On MI355X a plain
// three-read, one-write streaming kernel at B=1, L=8192, D=4096 (bf16, spans
// of 8 chunks, two in flight) took 48.8 us with 8 waves and 256-byte
// segments against 46.9 us with 16 waves and 512-byte segments.  A 16-wave
// workgroup has 128 VGPRs per lane: one chunk in flight (two spill), and for
// KH >= 2 the Toeplitz fragments are built from the staged tap pairs right
// before their MFMAs instead of being kept (48 VGPRs for KH = 4), with one
// staging tile (two would not fit the LDS).
constexpr int kWideWaves = 16;
constexpr int kWidePrefetch = 1;
constexpr int64_t kWideWorkgroups = 256;  // one 16-wave workgroup per CU (112 KiB of LDS)
// Longer filters take 16 waves from this many workgroups (4 per CU) on: the
// 16-wave form's matrix-core work is not hidden while every workgroup runs
// in one round.  Measured on MI355X, l_h = 128, D = 4096, per launch, 8 /
// 16 waves: B=1, L=8192 48.0 / 52.5 us; L=16384 93.5 / 96.0 (512
// workgroups); L=32768 195 / 185 (1024); L=65536 403 / 365; B=4, L=32768
// 808 / 720; L=2^20 6.43 / 5.72 ms.
constexpr int64_t kWideMrWorkgroups = 1024;
template <int KH, int... Ss> KernelFn wide_entry(int si, std::integer_sequence<int, Ss...>) {
    static constexpr KernelFn fns[] = {hyena_fwd_kernel<false, KH, kWidePrefetch, kSpans[Ss], false, false, kWideWaves>...};
    return fns[si];
}
KernelFn pick_wide(int kh, int si) {
    switch (kh) {
    case 0: return wide_entry<0>(si, std::make_integer_sequence<int, kNumSpans>{});
    case 1: return wide_entry<1>(si, std::make_integer_sequence<int, kNumSpans>{});
    case 2: return wide_entry<2>(si, std::make_integer_sequence<int, kNumSpans>{});
    case 3: return wide_entry<3>(si, std::make_integer_sequence<int, kNumSpans>{});
    default: return wide_entry<4>(si, std::make_integer_sequence<int, kNumSpans>{});
    }
}

template <bool F32, int Fam, int KH, int... Ss>
typename FnType<F32, Fam>::type span_table_entry(int si, std::integer_sequence<int, Ss...>) {
    static constexpr typename FnType<F32, Fam>::type fns[] = {kernel_of<F32, Fam, KH, kSpans[Ss]>()...};
    return fns[si];
}

template <bool F32, int Fam>
typename FnType<F32, Fam>::type pick_kernel(int kh, int si) {
    constexpr int n = kSpanCount<F32, Fam>;
    switch (kh) {
    case 0: return span_table_entry<F32, Fam, 0>(si, std::make_integer_sequence<int, n>{});
    case 1: return span_table_entry<F32, Fam, 1>(si, std::make_integer_sequence<int, n>{});
    case 2: return span_table_entry<F32, Fam, 2>(si, std::make_integer_sequence<int, n>{});
    case 3: return span_table_entry<F32, Fam, 3>(si, std::make_integer_sequence<int, n>{});
    default: return span_table_entry<F32, Fam, 4>(si, std::make_integer_sequence<int, n>{});
    }
}

constexpr int64_t kMaxWindowBytes = (int64_t)1 << 31;

struct Plan {
    int64_t span, n_spans, n_slabs, n_chunks, workgroups;
    int kh, span_index;
    bool wide = false;  // the 16-wave forward (256-channel slabs)
};

int check_sizes(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, int dtype) {
    if (dtype != HYENA_DTYPE_BF16 && dtype != HYENA_DTYPE_F32) return HYENA_ERR_DTYPE;
    if (B < 0 || L < 0 || D < 0) return HYENA_ERR_SHAPE;
    if (group_size < 1 || D % group_size != 0) return HYENA_ERR_GROUP;
    if (l_h < 1 || l_h > kMaxTaps) return HYENA_ERR_FILTER_LEN;
    // element count must fit comfortably in 63 bits
    if (B > 0 && L > 0 && D > 0) {
        const int64_t lim = INT64_MAX / 8;
        if (L > lim / D || B > lim / (L * D)) return HYENA_ERR_SHAPE;
    }
    return HYENA_OK;
}

int make_plan(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, int dtype,
              int64_t span_req, Plan *pl, int family = kFwd) {
    const int64_t eb = dtype == HYENA_DTYPE_F32 ? 4 : 2;
    pl->kh = (int)((l_h - 1 + 31) / 32);
    pl->n_chunks = (L + kChunk - 1) / kChunk;
    // 16 waves: always for SE; for longer filters once the grid has
    // kWideMrWorkgroups workgroups at 8-chunk spans (below that the 8-wave
    // kernel, which overlaps each chunk's epilogue with the next chunk's
    // MFMAs in a second staging tile, is faster)
    pl->wide = family == kFwd && dtype == HYENA_DTYPE_BF16 &&
               (pl->kh <= 1 || B * ((D + kTile * kWideWaves - 1) / (kTile * kWideWaves)) *
                                       ((pl->n_chunks + 7) / 8) >= kWideMrWorkgroups);
    pl->n_slabs = (D + (pl->wide ? kTile * kWideWaves : kSlab) - 1) / (pl->wide ? kTile * kWideWaves : kSlab);
    if (group_size % kTile != 0) return HYENA_ERR_UNSUPPORTED;
    if (D > INT32_MAX / 16) return HYENA_ERR_UNSUPPORTED;
    // Default span: long enough that the 32*KH history rows a workgroup
    // re-reads stay a small share of its rows (2*KH chunks: 1/4 at most),
    // short enough that many workgroups balance the CUs.  Measured on
    // MI355X at D=4096 (SE then MR, bf16): MR best at 8 chunks from L=8192
    // to 2^20.  The 16-wave SE kernel: spans up to 8 chunks while every CU
    // still gets a workgroup (kWideWorkgroups); at B=1 that is 2 chunks at
    // L=2048, 4 at 4096 and 8 from 8192 on, each the fastest (or within 1%
    // of it) in the step.
    int64_t want = span_req;
    if (want <= 0) {
        want = pl->kh <= 1 ? 2 : 2 * pl->kh;
        if (pl->wide) {
            want = 8;
            while (pl->kh <= 1 && want > 1 && B * pl->n_slabs * ((pl->n_chunks + want - 1) / want) < kWideWorkgroups) want /= 2;
        }
    }
    // the filter-gradient kernel writes one partial row per span: longer
    if (family == kDh && span_req <= 0) want = 16;
    if (want > pl->n_chunks) want = pl->n_chunks;
    // largest compiled span <= want whose byte window (history + span +
    // one chunk of slack) stays below 2^31
    int si = -1;
    const bool f32 = dtype == HYENA_DTYPE_F32;
    const int n_spans_compiled =
        family == kFwd ? (f32 ? kSpanCount<true, kFwd> : kSpanCount<false, kFwd>)
        : family == kRevDual ? (f32 ? kSpanCount<true, kRevDual> : kSpanCount<false, kRevDual>)
                             : (f32 ? kSpanCount<true, kDh> : kSpanCount<false, kDh>);
    for (int i = 0; i < n_spans_compiled; ++i) {
        const int64_t win = ((int64_t)kSpans[i] * kChunk + 32 * pl->kh + kChunk) * D * eb;
        if (win >= kMaxWindowBytes) break;
        if (i == 0 || kSpans[i] <= want) si = i;
    }
    if (si < 0) return HYENA_ERR_UNSUPPORTED;
    pl->span_index = si;
    pl->span = kSpans[si];
    pl->n_spans = (pl->n_chunks + pl->span - 1) / pl->span;
    pl->workgroups = pl->n_spans * pl->n_slabs * B;
    if (pl->workgroups > INT32_MAX || pl->n_spans > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
    return HYENA_OK;
}

// Plan of the chunk-direction kernel (group sizes not a multiple of 16).
// A workgroup owns CdTr::SLAB channels of one batch row and a span of
// 256-row blocks.  By default the spans are as long as it takes to make
// about as many workgroups as the CUs hold at once (kCdWorkgroups: 256 CUs,
// one 8-wave workgroup each), which reads the history rows and stages the
// taps once per span; `span_req` (in 64-row chunks) overrides.  `span` is reported in
// chunks.  Buffer windows are per block, so spans have no length limit.
constexpr int64_t kCdWorkgroups = 256 * (8 / kCdWaves);

int cd_plan(int64_t B, int64_t L, int64_t D, int64_t l_h, int dtype, int64_t span_req, Plan *pl) {
    const bool f32 = dtype == HYENA_DTYPE_F32;
    const int64_t eb = f32 ? 4 : 2;
    const int64_t slab = f32 ? CdTr<true>::SLAB : CdTr<false>::SLAB;
    if ((D * eb) % 16 != 0) return HYENA_ERR_UNSUPPORTED;  // 16-byte row segments
    if (D > INT32_MAX / 16 || (kCdBlock + 128) * D * eb >= kMaxWindowBytes) return HYENA_ERR_UNSUPPORTED;
    pl->kh = (int)((l_h - 1 + 31) / 32);
    pl->n_chunks = (L + kChunk - 1) / kChunk;
    const int64_t n_blocks = (L + kCdBlock - 1) / kCdBlock;
    pl->n_slabs = (D + slab - 1) / slab;
    int64_t sb = span_req > 0 ? (span_req * kChunk + kCdBlock - 1) / kCdBlock
                              : (n_blocks * pl->n_slabs * B + kCdWorkgroups - 1) / kCdWorkgroups;
    sb = max((int64_t)1, min(sb, n_blocks));
    pl->span_index = 0;
    pl->span = sb * (kCdBlock / kChunk);
    pl->n_spans = (n_blocks + sb - 1) / sb;
    pl->workgroups = pl->n_spans * pl->n_slabs * B;
    if (pl->workgroups > INT32_MAX || pl->n_spans > INT32_MAX || sb > INT32_MAX / kCdBlock)
        return HYENA_ERR_UNSUPPORTED;
    return HYENA_OK;
}

// Plan of the short-filter direct kernel (group sizes off the 16-channel
// tile, l_h <= kDirTaps).  One wave per 256-channel slab and span of rows;
// spans of 256 rows, halved down to 64 while that leaves fewer than 1024
// workgroups (four waves per CU) or a byte window (span + 16 rows) of 2^31
// or more, or span_req chunks.  `kh` holds the compiled tap count (1, 2, 4 or
// 8) and `span` the span in 64-row chunks.
constexpr int64_t kDirWorkgroups = 1024;

int dir_plan(int64_t B, int64_t L, int64_t D, int64_t l_h, int dtype, int64_t span_req, Plan *pl) {
    const int64_t eb = dtype == HYENA_DTYPE_F32 ? 4 : 2;
    if ((D * eb) % 16 != 0) return HYENA_ERR_UNSUPPORTED;  // same row rule as the chunk-direction kernel
    if (D > INT32_MAX / 16) return HYENA_ERR_UNSUPPORTED;
    pl->kh = l_h <= 1 ? 1 : l_h <= 2 ? 2 : l_h <= 4 ? 4 : 8;
    pl->n_chunks = (L + kChunk - 1) / kChunk;
    pl->n_slabs = (D + kDirSlab - 1) / kDirSlab;
    int64_t rows;
    if (span_req > 0) {
        rows = min(span_req, pl->n_chunks) * kChunk;
    } else {
        rows = 256;
        while (rows > kChunk && (B * pl->n_slabs * ((L + rows - 1) / rows) < kDirWorkgroups ||
                                 (rows + 2 * kDirTaps) * D * eb >= kMaxWindowBytes))
            rows /= 2;
    }
    // the windows: a span, the rows before it and (the backward) after it
    if ((rows + 2 * kDirTaps) * D * eb >= kMaxWindowBytes) return HYENA_ERR_UNSUPPORTED;
    pl->span_index = 0;
    pl->span = rows / kChunk;
    pl->n_spans = (L + rows - 1) / rows;
    pl->workgroups = pl->n_spans * pl->n_slabs * B;
    if (pl->workgroups > INT32_MAX || pl->n_spans > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
    return HYENA_OK;
}

template <bool F32, bool REV = false, bool DUAL = false> KernelFn pick_direct(int lh) {
    switch (lh) {
    case 1: return hyena_fwd_direct_kernel<F32, 1, REV, DUAL>;
    case 2: return hyena_fwd_direct_kernel<F32, 2, REV, DUAL>;
    case 4: return hyena_fwd_direct_kernel<F32, 4, REV, DUAL>;
    default: return hyena_fwd_direct_kernel<F32, 8, REV, DUAL>;
    }
}

template <bool F32> DhFn pick_lag(int ng2) {
    switch (ng2) {
    case 1: return hyena_bwd_dh_lag_kernel<F32, 1>;
    case 2: return hyena_bwd_dh_lag_kernel<F32, 2>;
    case 4: return hyena_bwd_dh_lag_kernel<F32, 4>;
    default: return hyena_bwd_dh_lag_kernel<F32, 8>;
    }
}

// Plan of the off-tile filter-gradient pass for filters over kDirTaps taps:
// kLagCh channels and kLagSpanRows rows (fewer for a shorter sequence) per
// workgroup; `kh` holds the tap groups of 16 the kernel sums (a power of 2,
// NG2) and `span` the span in 64-row chunks.
int lag_plan(int64_t B, int64_t L, int64_t D, int64_t l_h, int dtype, Plan *pl) {
    if (D > INT32_MAX / 16) return HYENA_ERR_UNSUPPORTED;
    const int ng = (int)((l_h + 15) / 16);
    pl->kh = ng <= 1 ? 1 : ng <= 2 ? 2 : ng <= 4 ? 4 : 8;
    pl->n_chunks = (L + kChunk - 1) / kChunk;
    // a span's byte window (its rows, or the 160 rows of history before it)
    // is addressed with 32-bit offsets: shorter spans for very wide rows
    const int64_t row_bytes = D * (dtype == HYENA_DTYPE_F32 ? 4 : 2);
    const int64_t fit = ((kMaxWindowBytes - 1) / row_bytes - 160) / kChunk * kChunk;
    if (fit < kChunk) return HYENA_ERR_UNSUPPORTED;
    const int64_t rows = min(min((int64_t)kLagSpanRows, fit), pl->n_chunks * kChunk);
    pl->span_index = 0;
    pl->span = rows / kChunk;
    pl->n_spans = (L + rows - 1) / rows;
    pl->n_slabs = (D + kLagCh - 1) / kLagCh;
    pl->workgroups = pl->n_spans * pl->n_slabs * B;
    if (pl->workgroups > INT32_MAX || B * pl->n_spans > INT32_MAX) return HYENA_ERR_UNSUPPORTED;
    return HYENA_OK;
}

template <bool F32> DhFn pick_direct_dh(int lh) {
    switch (lh) {
    case 1: return hyena_bwd_direct_kernel<F32, 1>;
    case 2: return hyena_bwd_direct_kernel<F32, 2>;
    case 4: return hyena_bwd_direct_kernel<F32, 4>;
    default: return hyena_bwd_direct_kernel<F32, 8>;
    }
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Fixed device scratch of the no-allocation backward: the partial filter
// gradients of pass 1 (one row of l_h floats per batch row, span and
// 16-channel tile, or per channel off the tile).  Every device the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is
// looked up once per device, with that device current, and only that
// address is used from then on.
constexpr int64_t kScratchBytes = (int64_t)16 << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The scratch array's address on the device `stream` belongs to (the
// current device for the null stream), or null if HIP reports an error.
void *scratch_on_stream_device(void *stream) {
    int dev = -1;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice((hipStream_t)stream, &d) != hipSuccess) return nullptr;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void *ptr = nullptr;
        const hipError_t rc = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
        if (rc != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int hyena_conv_plan(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, int dtype,
                    int64_t span_chunks, int64_t *span_out, int64_t *workgroups_out) {
    int st = check_sizes(B, L, D, group_size, l_h, dtype);
    if (st != HYENA_OK) return st;
    if (B == 0 || L == 0 || D == 0) {
        if (span_out) *span_out = 0;
        if (workgroups_out) *workgroups_out = 0;
        return HYENA_OK;
    }
    Plan pl;
    st = group_size % kTile == 0 ? make_plan(B, L, D, group_size, l_h, dtype, span_chunks, &pl)
         : l_h <= kDirTaps       ? dir_plan(B, L, D, l_h, dtype, span_chunks, &pl)
                                 : cd_plan(B, L, D, l_h, dtype, span_chunks, &pl);
    if (st != HYENA_OK) return st;
    if (span_out) *span_out = pl.span;
    if (workgroups_out) *workgroups_out = pl.workgroups;
    return HYENA_OK;
}

// Shared by every forward entry point: host checks, plan, launch.
static int fwd_launch(const void *q, const void *k, const void *v, const void *h, const void *kp,
                      const void *vp, int64_t P, int64_t B, int64_t L, int64_t D, int64_t group_size,
                      int64_t l_h, void *out, int dtype, int64_t span_chunks, void *stream) {
    int st = check_sizes(B, L, D, group_size, l_h, dtype);
    if (st != HYENA_OK) return st;
    if (P < 0) return HYENA_ERR_SHAPE;
    if (B == 0 || L == 0 || D == 0) return HYENA_OK;
    if (!q || !k || !v || !h || !out) return HYENA_ERR_NULL;
    if (P > 0 && (!kp || !vp)) return HYENA_ERR_NULL;
    const size_t eb = dtype == HYENA_DTYPE_F32 ? 4 : 2;
    uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
    if (P > 0) mis |= (uintptr_t)kp | (uintptr_t)vp;
    if (mis & 15u) return HYENA_ERR_ALIGN;
    if ((uintptr_t)h & (eb - 1)) return HYENA_ERR_ALIGN;
    const size_t nbytes = (size_t)B * (size_t)L * (size_t)D * eb;
    const size_t hbytes = (size_t)(D / group_size) * (size_t)l_h * eb;
    if (overlaps(out, nbytes, q, nbytes) || overlaps(out, nbytes, k, nbytes) ||
        overlaps(out, nbytes, v, nbytes) || overlaps(out, nbytes, h, hbytes))
        return HYENA_ERR_ALIAS;
    if (P > 0) {
        if (P > INT32_MAX / 4 || P * D * (int64_t)eb >= kMaxWindowBytes) return HYENA_ERR_UNSUPPORTED;
        const size_t pbytes = (size_t)B * (size_t)P * (size_t)D * eb;
        if (overlaps(out, nbytes, kp, pbytes) || overlaps(out, nbytes, vp, pbytes)) return HYENA_ERR_ALIAS;
    }
    const bool chunk_dir = group_size % kTile != 0;
    // off the 16-channel tile: a few taps are summed directly, longer
    // filters take the chunk-direction GEMMs (which take no history prefix)
    const bool direct = chunk_dir && l_h <= kDirTaps;
    Plan pl;
    st = direct      ? dir_plan(B, L, D, l_h, dtype, span_chunks, &pl)
         : chunk_dir ? cd_plan(B, L, D, l_h, dtype, span_chunks, &pl)
                     : make_plan(B, L, D, group_size, l_h, dtype, span_chunks, &pl);
    if (st != HYENA_OK) return st;

    Params p;
    p.q = q; p.k = k; p.v = v; p.h = h; p.y = out;
    p.kp = P > 0 ? kp : nullptr;
    p.vp = P > 0 ? vp : nullptr;
    p.L = L;
    p.D = (int32_t)D;
    p.group_size = (int32_t)group_size;
    p.l_h = (int32_t)l_h;
    p.n_spans = (int32_t)pl.n_spans;
    p.n_slabs = (int32_t)pl.n_slabs;
    p.P = (int32_t)P;
    p.span_blocks = (int32_t)(pl.span / (kCdBlock / kChunk));
    p.span_rows = (int32_t)(pl.span * kChunk);
    p.g2 = nullptr;
    p.y2 = nullptr;
    const bool f32 = dtype == HYENA_DTYPE_F32;
    KernelFn fn = direct      ? (f32 ? pick_direct<true>(pl.kh) : pick_direct<false>(pl.kh))  // (reads kp, vp when P > 0)
                  : chunk_dir ? (f32 ? pick_kernel<true, kCd>(pl.kh, pl.span_index)
                                     : pick_kernel<false, kCd>(pl.kh, pl.span_index))
                  : pl.wide   ? pick_wide(pl.kh, pl.span_index)
                              : (f32 ? pick_kernel<true, kFwd>(pl.kh, pl.span_index)
                                     : pick_kernel<false, kFwd>(pl.kh, pl.span_index));
    const int threads = direct ? 64 : chunk_dir ? kCdThreads : pl.wide ? 64 * kWideWaves : kThreads;
    hipLaunchKernelGGL(fn, dim3((unsigned)pl.workgroups), dim3(threads), 0,
                       (hipStream_t)stream, p);
    if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
    return HYENA_OK;
}

// Partial-row count of the filter-gradient pass 1 (one row per span per
// batch row), for the workspace size.  Group sizes off the 16-channel tile
// take the direct kernels (filters of at most kDirTaps taps; one partial row
// per span per batch row and channel), else the grouped ones.
static int dh_plan(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, int dtype,
                   Plan *pl, int64_t *ws_bytes) {
    if (group_size % kTile != 0) {
        int st = l_h <= kDirTaps ? dir_plan(B, L, D, l_h, dtype, 0, pl) : lag_plan(B, L, D, l_h, dtype, pl);
        if (st != HYENA_OK) return st;
        if ((D * (dtype == HYENA_DTYPE_F32 ? 4 : 2)) % 16 != 0) return HYENA_ERR_UNSUPPORTED;
        *ws_bytes = B * pl->n_spans * D * l_h * (int64_t)sizeof(float);
        return HYENA_OK;
    }
    int st = make_plan(B, L, D, group_size, l_h, dtype, 0, pl, kDh);
    if (st != HYENA_OK) return st;
    *ws_bytes = B * pl->n_spans * (D / kTile) * l_h * (int64_t)sizeof(float);
    return HYENA_OK;
}

int hyena_conv_fwd_ex(const void *q, const void *k, const void *v, const void *h, int64_t B,
                      int64_t L, int64_t D, int64_t group_size, int64_t l_h, void *out, int dtype,
                      int64_t span_chunks, void *stream) {
    return fwd_launch(q, k, v, h, nullptr, nullptr, 0, B, L, D, group_size, l_h, out, dtype,
                      span_chunks, stream);
}

int hyena_conv_fwd_halo(const void *q, const void *k, const void *v, const void *h,
                        const void *k_prev, const void *v_prev, int64_t P, int64_t B, int64_t L,
                        int64_t D, int64_t group_size, int64_t l_h, void *out, int dtype,
                        int64_t span_chunks, void *stream) {
    return fwd_launch(q, k, v, h, k_prev, v_prev, P, B, L, D, group_size, l_h, out, dtype,
                      span_chunks, stream);
}

int hyena_conv_bwd_workspace(int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h,
                             int dtype, int64_t *bytes_out) {
    int st = check_sizes(B, L, D, group_size, l_h, dtype);
    if (st != HYENA_OK) return st;
    if (!bytes_out) return HYENA_ERR_NULL;
    if (B == 0 || L == 0 || D == 0) {
        *bytes_out = 0;
        return HYENA_OK;
    }
    Plan pl;
    return dh_plan(B, L, D, group_size, l_h, dtype, &pl, bytes_out);
}

// The backward of both entry points.  `scratch` set: the partial filter
// gradients go to this library's fixed device array instead of `workspace`
// (which is then ignored); its address on the stream's device is looked up
// only after every host check has passed.
static int bwd_entry(const void *q, const void *k, const void *v, const void *h, const void *dy,
                     int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, void *dq,
                     void *dk, void *dv, float *dh, void *workspace, int64_t workspace_bytes,
                     int dtype, void *stream, bool scratch) {
    int st = check_sizes(B, L, D, group_size, l_h, dtype);
    if (st != HYENA_OK) return st;
    if (!q || !k || !v || !h || !dy) return HYENA_ERR_NULL;
    if ((dk == nullptr) != (dv == nullptr)) return HYENA_ERR_NULL;
    const size_t eb = dtype == HYENA_DTYPE_F32 ? 4 : 2;
    const size_t nbytes = (size_t)B * (size_t)L * (size_t)D * eb;
    const size_t hbytes = (size_t)(D / group_size) * (size_t)l_h * eb;
    const size_t dhbytes = (size_t)(D / group_size) * (size_t)l_h * sizeof(float);
    uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)dy;
    if (dq) mis |= (uintptr_t)dq;
    if (dk) mis |= (uintptr_t)dk | (uintptr_t)dv;
    if (mis & 15u) return HYENA_ERR_ALIGN;
    if (scratch) workspace = nullptr;
    if (((uintptr_t)h & (eb - 1)) || ((uintptr_t)dh & 3u) || ((uintptr_t)workspace & 15u))
        return HYENA_ERR_ALIGN;
    // every output and the workspace are disjoint from every input and
    // from each other
    const void *in[5] = {q, k, v, dy, h};
    const size_t in_n[5] = {nbytes, nbytes, nbytes, nbytes, hbytes};
    Plan dpl;
    int64_t ws_need = 0;
    if (B > 0 && L > 0 && D > 0) {
        st = dh_plan(B, L, D, group_size, l_h, dtype, &dpl, &ws_need);
        if (st != HYENA_OK) return st;
    }
    const void *out[5] = {dq, dk, dv, dh, dh ? workspace : nullptr};
    const size_t out_n[5] = {nbytes, nbytes, nbytes, dhbytes, (size_t)ws_need};
    for (int i = 0; i < 5; ++i) {
        if (!out[i]) continue;
        for (int j = 0; j < 5; ++j)
            if (overlaps(out[i], out_n[i], in[j], in_n[j])) return HYENA_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (out[j] && overlaps(out[i], out_n[i], out[j], out_n[j])) return HYENA_ERR_ALIAS;
    }
    if (scratch) {
        if (dh && ws_need > kScratchBytes) return HYENA_ERR_SCRATCH;
        if (dh && ws_need > 0) {
            workspace = scratch_on_stream_device(stream);
            if (!workspace) return HYENA_ERR_LAUNCH;
        }
    } else if (dh && (!workspace || workspace_bytes < ws_need)) {
        return HYENA_ERR_WORKSPACE;
    }
    if (B == 0 || L == 0 || D == 0) {
        // no rows: dh is zero (D == 0: dh has no elements)
        const int64_t n = (int64_t)(dhbytes / sizeof(float));
        if (dh && n > 0) {
            hipLaunchKernelGGL(hyena_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               (hipStream_t)stream, dh, n);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        }
        return HYENA_OK;
    }
    const bool f32 = dtype == HYENA_DTYPE_F32;
    if (group_size % kTile != 0 && l_h > kDirTaps) {
        // longer filters off the tile: dq is the chunk-direction forward with
        // dy as the gate; dk and dv the same walked backwards in time (x =
        // dy q, gated by v and by k); dh the lag products per channel and the
        // per-group reduction
        if (dq) {
            st = fwd_launch(dy, k, v, h, nullptr, nullptr, 0, B, L, D, group_size, l_h, dq, dtype, 0, stream);
            if (st != HYENA_OK) return st;
        }
        if (dk) {
            Plan pl;
            st = cd_plan(B, L, D, l_h, dtype, 0, &pl);
            if (st != HYENA_OK) return st;
            Params p;
            p.q = v; p.k = dy; p.v = q; p.h = h; p.y = dk;
            p.g2 = k; p.y2 = dv;
            p.kp = nullptr; p.vp = nullptr; p.P = 0;
            p.span_blocks = (int32_t)(pl.span / (kCdBlock / kChunk));
            p.span_rows = (int32_t)(pl.span * kChunk);
            p.L = L;
            p.D = (int32_t)D;
            p.group_size = (int32_t)group_size;
            p.l_h = (int32_t)l_h;
            p.n_spans = (int32_t)pl.n_spans;
            p.n_slabs = (int32_t)pl.n_slabs;
            KernelFn fn = f32 ? pick_kernel<true, kCdRevDual>(pl.kh, 0) : pick_kernel<false, kCdRevDual>(pl.kh, 0);
            hipLaunchKernelGGL(fn, dim3((unsigned)pl.workgroups), dim3(kCdThreads), 0, (hipStream_t)stream, p);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        }
        if (dh) {
            DhParams p;
            p.q = q; p.k = k; p.v = v; p.dy = dy;
            p.ws = (float *)workspace;
            p.h = h;
            p.dq = nullptr; p.dk = nullptr; p.dv = nullptr;
            p.L = L;
            p.D = (int32_t)D;
            p.l_h = (int32_t)l_h;
            p.n_spans = (int32_t)dpl.n_spans;
            p.n_slabs = (int32_t)dpl.n_slabs;
            p.group_size = (int32_t)group_size;
            p.span_rows = (int32_t)(dpl.span * kChunk);
            DhFn fn = f32 ? pick_lag<true>(dpl.kh) : hyena_bwd_dh_lag_mfma_kernel;
            hipLaunchKernelGGL(fn, dim3((unsigned)dpl.workgroups), dim3(512), 0, (hipStream_t)stream, p);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
            const int G = (int)(D / group_size);
            const int n = G * (int)l_h;
            hipLaunchKernelGGL(hyena_bwd_direct_dh_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               (hipStream_t)stream, (const float *)workspace, dh, (int)(B * dpl.n_spans), (int)D,
                               (int)group_size, (int)l_h, G);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        }
        return HYENA_OK;
    }
    if (group_size % kTile != 0) {
        // short filters off the tile: the direct kernels, with the direct
        // forward's plan
        if (dh) {
            // the whole backward in one walk (any of dq, dk, dv may be absent)
            DhParams p;
            p.q = q; p.k = k; p.v = v; p.dy = dy;
            p.ws = (float *)workspace;
            p.h = h;
            p.dq = dq;
            p.dk = dk; p.dv = dv;
            p.L = L;
            p.D = (int32_t)D;
            p.l_h = (int32_t)l_h;
            p.n_spans = (int32_t)dpl.n_spans;
            p.n_slabs = (int32_t)dpl.n_slabs;
            p.group_size = (int32_t)group_size;
            p.span_rows = (int32_t)(dpl.span * kChunk);
            DhFn fn = f32 ? pick_direct_dh<true>(dpl.kh) : pick_direct_dh<false>(dpl.kh);
            hipLaunchKernelGGL(fn, dim3((unsigned)dpl.workgroups), dim3(64), 0, (hipStream_t)stream, p);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        } else if (dq) {
            st = fwd_launch(dy, k, v, h, nullptr, nullptr, 0, B, L, D, group_size, l_h, dq, dtype, 0, stream);
            if (st != HYENA_OK) return st;
        }
        if (dk && !dh) {
            // dx walked backwards in time with x = dy q, gated by v and k
            Params p;
            p.q = v; p.k = dy; p.v = q; p.h = h; p.y = dk;
            p.g2 = k; p.y2 = dv;
            p.kp = nullptr; p.vp = nullptr; p.P = 0; p.span_blocks = 0;
            p.span_rows = (int32_t)(dpl.span * kChunk);
            p.L = L;
            p.D = (int32_t)D;
            p.group_size = (int32_t)group_size;
            p.l_h = (int32_t)l_h;
            p.n_spans = (int32_t)dpl.n_spans;
            p.n_slabs = (int32_t)dpl.n_slabs;
            KernelFn fn = f32 ? pick_direct<true, true, true>(dpl.kh) : pick_direct<false, true, true>(dpl.kh);
            hipLaunchKernelGGL(fn, dim3((unsigned)dpl.workgroups), dim3(64), 0, (hipStream_t)stream, p);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        }
        if (dh) {
            const int G = (int)(D / group_size);
            const int n = G * (int)l_h;
            hipLaunchKernelGGL(hyena_bwd_direct_dh_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               (hipStream_t)stream, (const float *)workspace, dh, (int)(B * dpl.n_spans), (int)D,
                               (int)group_size, (int)l_h, G);
            if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        }
        return HYENA_OK;
    }
    // bf16 with all four gradients: one kernel computes dq, dk, dv and the
    // partial dh, when its window (history, span, the rows its walk reads
    // past the span and a chunk of slack) stays below 2^31 bytes; else, with
    // dq and dh, one kernel computes both (below)
    const int64_t fut_rows = ((32 * (int64_t)dpl.kh + kChunk - 1) / kChunk) * kChunk;
    const bool fused_all = dq && dk && dv && dh && !f32 &&
                           (dpl.span * kChunk + 32 * dpl.kh + fut_rows + kChunk) * D * (int64_t)eb < kMaxWindowBytes;
    const bool fused_dq = dq && dh && !f32;

    // dq = dy * (h * (k v)): the forward with dy as the gate
    if (dq && !fused_dq) {
        st = fwd_launch(dy, k, v, h, nullptr, nullptr, 0, B, L, D, group_size, l_h, dq, dtype, 0, stream);
        if (st != HYENA_OK) return st;
    }
    // dk = v * dx, dv = k * dx with dx = h applied to dz = dy q at later rows:
    // the forward walked backwards in time, x = dy q, gates v and k
    if (dk && !fused_all) {
        Plan pl;
        st = make_plan(B, L, D, group_size, l_h, dtype, 0, &pl, kRevDual);
        if (st != HYENA_OK) return st;
        Params p;
        p.q = v; p.k = dy; p.v = q; p.h = h; p.y = dk;
        p.g2 = k; p.y2 = dv;
        p.kp = nullptr; p.vp = nullptr; p.P = 0; p.span_blocks = 0; p.span_rows = 0;
        p.L = L;
        p.D = (int32_t)D;
        p.group_size = (int32_t)group_size;
        p.l_h = (int32_t)l_h;
        p.n_spans = (int32_t)pl.n_spans;
        p.n_slabs = (int32_t)pl.n_slabs;
        KernelFn fn = f32 ? pick_kernel<true, kRevDual>(pl.kh, pl.span_index)
                          : pick_kernel<false, kRevDual>(pl.kh, pl.span_index);
        hipLaunchKernelGGL(fn, dim3((unsigned)pl.workgroups), dim3(kThreads), 0, (hipStream_t)stream, p);
        if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
    }
    // dh: partial sums per span (pass 1, with dq when fused), then their
    // reduction (pass 2)
    if (dh) {
        DhParams p;
        p.q = q; p.k = k; p.v = v; p.dy = dy;
        p.ws = (float *)workspace;
        p.h = h;
        p.dq = fused_dq ? dq : nullptr;
        p.dk = fused_all ? dk : nullptr;
        p.dv = fused_all ? dv : nullptr;
        p.span_rows = 0;
        p.L = L;
        p.D = (int32_t)D;
        p.l_h = (int32_t)l_h;
        p.n_spans = (int32_t)dpl.n_spans;
        p.n_slabs = (int32_t)dpl.n_slabs;
        p.group_size = (int32_t)group_size;
        DhFn fn = fused_all  ? pick_kernel<false, kBwd>(dpl.kh, dpl.span_index)
                  : fused_dq ? pick_kernel<false, kDqDh>(dpl.kh, dpl.span_index)
                  : f32    ? pick_kernel<true, kDh>(dpl.kh, dpl.span_index)
                           : pick_kernel<false, kDh>(dpl.kh, dpl.span_index);
        hipLaunchKernelGGL(fn, dim3((unsigned)dpl.workgroups), dim3(kThreads), 0, (hipStream_t)stream, p);
        if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
        const int G = (int)(D / group_size);
        const int n = G * (int)l_h;
        hipLaunchKernelGGL(hyena_bwd_dh_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           (hipStream_t)stream, (const float *)workspace, dh, (int)(B * dpl.n_spans),
                           (int)(D / kTile), (int)(group_size / kTile), (int)l_h, G);
        if (hipGetLastError() != hipSuccess) return HYENA_ERR_LAUNCH;
    }
    return HYENA_OK;
}

int hyena_conv_bwd(const void *q, const void *k, const void *v, const void *h, const void *dy,
                   int64_t B, int64_t L, int64_t D, int64_t group_size, int64_t l_h, void *dq,
                   void *dk, void *dv, float *dh, void *workspace, int64_t workspace_bytes,
                   int dtype, void *stream) {
    return bwd_entry(q, k, v, h, dy, B, L, D, group_size, l_h, dq, dk, dv, dh, workspace,
                     workspace_bytes, dtype, stream, false);
}

int hyena_conv_bwd_noalloc(const void *q, const void *k, const void *v, const void *h,
                           const void *dy, int64_t B, int64_t L, int64_t D, int64_t group_size,
                           int64_t l_h, void *dq, void *dk, void *dv, float *dh, int dtype,
                           void *stream) {
    return bwd_entry(q, k, v, h, dy, B, L, D, group_size, l_h, dq, dk, dv, dh, nullptr, 0, dtype,
                     stream, true);
}

int64_t hyena_conv_scratch_bytes(void) { return kScratchBytes; }

int hyena_conv_fwd(const void *q, const void *k, const void *v, const void *h, int64_t B, int64_t L,
                   int64_t D, int64_t group_size, int64_t l_h, void *out, void *stream) {
    return hyena_conv_fwd_ex(q, k, v, h, B, L, D, group_size, l_h, out, HYENA_DTYPE_BF16, 0, stream);
}

int hyena_conv_fwd_f32(const void *q, const void *k, const void *v, const void *h, int64_t B,
                       int64_t L, int64_t D, int64_t group_size, int64_t l_h, void *out,
                       void *stream) {
    return hyena_conv_fwd_ex(q, k, v, h, B, L, D, group_size, l_h, out, HYENA_DTYPE_F32, 0, stream);
}

const char *hyena_conv_strerror(int status) {
    switch (status) {
    case HYENA_OK: return "ok";
    case HYENA_ERR_NULL: return "a required pointer is NULL";
    case HYENA_ERR_SHAPE: return "B, L or D is negative or the sizes overflow";
    case HYENA_ERR_GROUP: return "group_size must be >= 1 and divide D";
    case HYENA_ERR_FILTER_LEN: return "l_h must be in [1, 128]";
    case HYENA_ERR_ALIGN: return "q, k, v and out must be 16-byte aligned; h element aligned";
    case HYENA_ERR_ALIAS: return "out overlaps an input";
    case HYENA_ERR_UNSUPPORTED: return "unsupported case (off the 16-channel grouping rows must be a multiple of 16 bytes; long filters: D must be even and the transform at most 2^22 points; or the shape is too large to address)";
    case HYENA_ERR_LAUNCH: return "kernel launch failed";
    case HYENA_ERR_DTYPE: return "unknown dtype code";
    case HYENA_ERR_WORKSPACE: return "workspace missing or smaller than hyena_conv_bwd_workspace reports";
    case HYENA_ERR_SCRATCH: return "the problem needs more scratch than the no-allocation entry point's fixed device array holds (hyena_conv_scratch_bytes)";
    default: return "unknown status";
    }
}

int hyena_conv_block_len(void) { return kChunk; }

}  // extern "C"
