// Binary block mask builder (Binary Block Masking, "Presentation" and "How it
// works"): bit 0 of entry (b, i, j) is 1 when query tile i x key tile j of
// batch entry b holds at least one valid element; bit 1 marks a full tile (the
// whole tile inside [0, n) x [0, n) with every element valid), where the
// attention kernels need no element mask.  One matrix per batch entry, shared
// by every head and layer.
//
// Padding-only batches use the closed form (i*bq < n) && (j*bk < n), and
// ((i+1)*bq <= n) && ((j+1)*bk <= n) for full tiles, one wave per block row.
// With an element mask the builder is one HBM scan of the valid rectangle
// [0, n) x [0, n) of each mask: a workgroup owns a band of bq rows and a group
// of key tiles, so it writes its outputs alone (no atomics to global memory),
// and each wave walks one row at a time with 16-byte loads.
#include "device_common.h"
#include "kernels.h"

namespace sigattn {

// Grid: (Tq, B); one wave per block row i of batch entry b, its lanes
// stepping over the row's Tk entries.  The full-tile tests are written as
// i*bq <= n - bq (that is, (i+1)*bq <= n) so that no product passes L.
__global__ void __launch_bounds__(64)
blockmask_padding_kernel(const int32_t *__restrict__ seq_lens, int L, int bq, int bk, int Tq,
                         int Tk, uint8_t *__restrict__ out) {
    const int i = blockIdx.x, b = blockIdx.y;
    const int n = clamp_len(seq_lens[b], L);
    const bool row_any = i * bq < n, row_full = i * bq <= n - bq;
    uint8_t *row = out + ((int64_t)b * Tq + i) * Tk;
    for (int j = (int)threadIdx.x; j < Tk; j += 64) {
        const bool any = row_any && j * bk < n;
        const bool full = row_full && j * bk <= n - bk;
        row[j] = (uint8_t)(any | (full << 1));
    }
}

// Grid: (Tq * groups, B); 256 threads.  tiles_per_group * bk <= 1024 columns,
// and tiles_per_group <= 32 so one 32-bit word holds the group's flags.
__global__ void __launch_bounds__(256)
blockmask_scan_kernel(const int32_t *__restrict__ seq_lens, const uint8_t *__restrict__ mask,
                      int L, int bq, int bk_shift, int Tq, int Tk, int tiles_per_group,
                      int groups, uint8_t *__restrict__ out) {
    __shared__ uint32_t flags, zeros;  // per key tile: a valid element seen / an invalid one
    const int b = blockIdx.y;
    const int i = blockIdx.x / groups;
    const int g = blockIdx.x % groups;
    const int j0 = g * tiles_per_group;
    const int j1 = min(j0 + tiles_per_group, Tk);
    const int n = clamp_len(seq_lens[b], L);
    const int r_lo = i * bq, r_hi = min(min(r_lo + bq, L), n);
    const int c_lo = j0 << bk_shift, c_hi = min(j1 << bk_shift, n);
    if (threadIdx.x == 0) flags = zeros = 0u;
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t total = (uint64_t)gridDim.y * (uint64_t)L * (uint64_t)L;
    uint32_t bits = 0, zbits = 0;
    // One 16-byte chunk at byte address a of row `row` (columns [lo, hi) of
    // the scan): non-zero bytes mark their tile kept, zero bytes not full.
    auto chunk = [&](uint4 u, uint64_t a, uint64_t row, uint64_t lo, uint64_t hi) {
        const uint32_t nz = u.x | u.y | u.z | u.w;
        const uint64_t s0 = a > lo ? a : lo, s1 = a + 16 < hi ? a + 16 : hi;  // in-range part
        const int t0 = (int)((s0 - row) >> bk_shift) - j0;
        const int t1 = (int)((s1 - 1 - row) >> bk_shift) - j0;
        if (nz == 0u) {  // every byte invalid
            zbits |= (1u << t0) | (1u << t1);
            return;
        }
        const uint32_t zero_byte = ((u.x - 0x01010101u) & ~u.x) | ((u.y - 0x01010101u) & ~u.y) |
                                   ((u.z - 0x01010101u) & ~u.z) | ((u.w - 0x01010101u) & ~u.w);
        if ((zero_byte & 0x80808080u) == 0u) {  // every byte valid: its tile(s) kept
            bits |= (1u << t0) | (1u << t1);
            return;
        }
        // Mixed chunk: one bit per byte (non-zero), bit-parallel.
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        uint32_t nz16 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // Bit 7 of each non-zero byte, moved to four adjacent bits.
            const uint32_t m = (((w[q] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w[q]) & 0x80808080u;
            nz16 |= (((m >> 7) * 0x00204081u) >> 21 & 0xfu) << (4 * q);
        }
        const int s = (int)(s0 - a), e = (int)(s1 - a);  // in-range bytes [s, e)
        const uint32_t range16 = ((1u << e) - 1u) & ~((1u << s) - 1u);
        // Bytes before the start of tile t1 belong to tile t0.
        const int64_t split = (int64_t)(((uint64_t)(t1 + j0) << bk_shift) + row) - (int64_t)a;
        const uint32_t first = t1 == t0 ? 0xffffu : (1u << split) - 1u;
        const uint32_t in0 = range16 & first, in1 = range16 & ~first;
        if (nz16 & in0) bits |= 1u << t0;
        if (nz16 & in1) bits |= 1u << t1;
        if (~nz16 & in0) zbits |= 1u << t0;
        if (~nz16 & in1) zbits |= 1u << t1;
    };
    if (r_lo < r_hi && c_lo < c_hi) {
        // Four rows per wave in flight: all their loads are issued before any
        // is examined (eight rows measured slower).  A row's window of at
        // most 1024 columns, aligned down to 16 bytes, spans at most 65
        // chunks: lane l takes chunks l and l + 64, both loaded up front so
        // no lane waits on a second round trip.  Chunks that would run past
        // the end of the mask are read byte by byte (bytes past the end 0).
        for (int rb = r_lo + wave; rb < r_hi; rb += 16) {
            uint4 u[4][2];
            uint64_t arow[4], alo[4], ahi[4], a0[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = rb + 4 * t;
                arow[t] = ((uint64_t)b * L + (r < r_hi ? r : r_lo)) * (uint64_t)L;
                alo[t] = arow[t] + c_lo;
                ahi[t] = r < r_hi ? arow[t] + c_hi : 0;  // rows past r_hi: nothing
                a0[t] = (alo[t] & ~(uint64_t)15) + 16u * lane;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const uint64_t a = a0[t] + 1024u * k;
                    u[t][k] = make_uint4(0u, 0u, 0u, 0u);
                    if (a < ahi[t] && a + 16 <= total)
                        u[t][k] = *reinterpret_cast<const uint4 *>(mask + a);
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const uint64_t a = a0[t] + 1024u * k;
                    if (a >= ahi[t]) continue;
                    uint4 v = u[t][k];
                    if (a + 16 > total) {
                        uint8_t bb[16];
                        for (int e = 0; e < 16; ++e) bb[e] = (a + e < total) ? mask[a + e] : 0;
                        v = *reinterpret_cast<const uint4 *>(bb);
                    }
                    chunk(v, a, arow[t], alo[t], ahi[t]);
                }
        }
    }
    if (bits) atomicOr(&flags, bits);
    if (zbits) atomicOr(&zeros, zbits);
    __syncthreads();
    const int t = threadIdx.x;
    if (t < j1 - j0) {
        // Full: the whole bq x bk tile inside [0, n)^2 and no invalid element.
        const bool inside = (i + 1) * bq <= n && ((j0 + t + 1) << bk_shift) <= n;
        const uint32_t any = (flags >> t) & 1u;
        const uint32_t full = inside && !((zeros >> t) & 1u) ? 1u : 0u;
        out[((int64_t)b * Tq + i) * Tk + j0 + t] = (uint8_t)(any | (full << 1));
    }
}

// Key-range masks: query row r keeps keys [lo_r, hi_r] within [0, n).  One
// workgroup per (query tile i, batch entry b) reads the tile's ranges into
// LDS once; each thread then decides its key tiles from the bq ranges alone
// (a tile is kept when some row's range meets it, full when it lies inside
// [0, n)^2 and every row's range covers it).  O(bq) work per entry, no mask.
__global__ void __launch_bounds__(256)
blockmask_range_kernel(const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ key_range,
                       int L, int bq, int bk, int Tq, int Tk, uint8_t *__restrict__ out) {
    __shared__ int2 rr[128];
    const int b = blockIdx.y, i = blockIdx.x;
    const int n = clamp_len(seq_lens[b], L);
    const int r0 = i * bq, rows = min(bq, L - r0);
    for (int t = threadIdx.x; t < rows; t += blockDim.x) {
        int2 v = make_int2(1, 0);  // empty: rows at or past n keep nothing
        if (r0 + t < n) {
            const int2 kr = reinterpret_cast<const int2 *>(key_range)[(int64_t)b * L + r0 + t];
            v = make_int2(max(kr.x, 0), min(kr.y, n - 1));
        }
        rr[t] = v;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < Tk; j += blockDim.x) {
        const int c0 = j * bk, c1 = c0 + bk - 1;
        bool any = false, full = (i + 1) * bq <= n && (j + 1) * bk <= n;
        for (int t = 0; t < rows; ++t) {
            const int2 v = rr[t];
            any = any || (v.x <= v.y && v.x <= c1 && v.y >= c0);
            full = full && v.x <= c0 && v.y >= c1;
        }
        out[((int64_t)b * Tq + i) * Tk + j] = (uint8_t)(any | (full << 1));
    }
}

hipError_t launch_blockmask(const int32_t *seq_lens, const uint8_t *mask,
                            const int32_t *key_range, int B, int L, int block_q, int block_k,
                            uint8_t *out, hipStream_t stream) {
    const int Tq = (int)(((int64_t)L + block_q - 1) / block_q);
    const int Tk = (int)(((int64_t)L + block_k - 1) / block_k);
    if (key_range != nullptr) {
        hipLaunchKernelGGL(blockmask_range_kernel, dim3((unsigned)Tq, (unsigned)B), dim3(256), 0,
                           stream, seq_lens, key_range, L, block_q, block_k, Tq, Tk, out);
        return hipGetLastError();
    }
    if (mask == nullptr) {
        hipLaunchKernelGGL(blockmask_padding_kernel, dim3((unsigned)Tq, (unsigned)B), dim3(64), 0,
                           stream, seq_lens, L, block_q, block_k, Tq, Tk, out);
        return hipGetLastError();
    }
    int bk_shift = 0;
    while ((1 << bk_shift) < block_k) ++bk_shift;
    const int tiles_per_group = 1024 / block_k;  // 8, 16 or 32 tiles: 1 KiB of each row
    const int groups = (Tk + tiles_per_group - 1) / tiles_per_group;
    hipLaunchKernelGGL(blockmask_scan_kernel, dim3((unsigned)(Tq * groups), (unsigned)B),
                       dim3(256), 0, stream, seq_lens, mask, L, block_q, bk_shift, Tq, Tk,
                       tiles_per_group, groups, out);
    return hipGetLastError();
}

}  // namespace sigattn
