// Work schedule of one batch, built once next to its block mask and shared by
// every head, by the forward and the backward launches, and by every layer
// with the same lengths and mask (Binary Block Masking, "Presentation": the
// block structure is computed once, in parallel, before the attention
// kernels; "How it works": the kernels then visit only the runs of kept
// blocks).  Two parts, laid out by schedule_layout (kernels.h):
//
// * Work items.  Workgroup i of an attention launch runs on XCD i % 8 and
//   reads its item from slot i, so XCD x works through the (length rank,
//   head) pairs x, x + 8, ... (all tiles of a pair share that XCD's L2; with
//   H a multiple of 8 every XCD gets one head of each batch entry), longest
//   sequence first (longest processing time first), and zero items: for its
//   pairs again, the fully padded tiles (all tiles of an empty sequence) in
//   runs of kZeroTiles, which only write zeros, so that the longest items
//   do not also carry their sequence's zero stores.  The forward's zero items
//   come after its compute items, where they fill the slots the launch's
//   tail leaves idle, unless they outnumber them (large padding): then they
//   are spread evenly between them, since dealt last they would form a burst
//   of pure writes that lengthens the launch.  The one-launch backward's,
//   with three times the zeros to write, are spread evenly over the second
//   half of its compute items.  Without a schedule every workgroup
//   derives its item from seq_lens itself (a rank of the lengths and prefix
//   sums over the pairs: several microseconds per workgroup), and the tiles
//   with valid rows write their sequence's padded tiles.
// * Kept-entry lists.  Per batch entry and 128-row group of queries (the
//   rows one forward or dQ workgroup owns) the block-mask entries that some
//   block row of the group keeps, with which rows keep it and which mark it
//   full; per 128-key group the same down the block columns (dK/dV).  The
//   kernels read their tiles from the list instead of scanning block-mask
//   lines for non-zero entries.
// For a padding-only batch the block mask is a closed form of the lengths,
// so the same launch writes it too.
#include "device_common.h"
#include "kernels.h"

namespace sigattn {

namespace {

constexpr int kSchedThreads = 256;
constexpr int kSortMax = 1024;  // larger batches keep their natural order

// Exclusive prefix sum over the workgroup's 256 threads; *total receives the
// sum.  Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int *wave_tot, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kSchedThreads / 64; ++i) {
        const int t = wave_tot[i];
        before += i < w ? t : 0;
        all += t;
    }
    __syncthreads();  // wave_tot is reused by the next call
    *total = all;
    return before + incl - v;
}

// floor(a / b) for 0 <= a < 2^48 and 0 < b < 2^31, exact: the fp64 quotient
// of two exactly represented operands is within 2^-5 of a / b, so its
// truncation is off by at most one and one integer test corrects it (a 64-bit
// integer division would be a long software sequence per item).
__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
    int64_t q = (int64_t)((double)a / (double)b);
    if (q * b > a)
        --q;
    else if ((q + 1) * b <= a)
        ++q;
    return q;
}

}  // namespace

// Block-mask entry (i, j) of a padding-only batch entry of length n: bit 0
// when the tile holds a valid element, bit 1 when it lies inside [0, n)^2.
// The full-tile tests are written as i*bq <= n - bq so no product passes L.
__device__ __forceinline__ uint32_t padding_entry(int i, int j, int n, int bq, int bk) {
    const bool any = i * bq < n && j * bk < n;
    const bool full = i * bq <= n - bq && j * bk <= n - bk;
    return (any ? 1u : 0u) | (full ? 2u : 0u);
}

// Grid: 16 item workgroups (XCD x = blockIdx.x % 8; blockIdx.x / 8 selects
// the one-kind array items1 or the two-kind array items2), then one wave per
// (direction, batch entry, group) for the entry lists, then, for a
// padding-only batch (bm_out given), one wave per block row writing the
// block mask, whose entries the lists then take from the same closed form
// instead of reading bm: the whole build is one launch.
__global__ void __launch_bounds__(kSchedThreads)
schedule_kernel(const int32_t *__restrict__ seq_lens, const uint8_t *__restrict__ bm, int B,
                int H, int L, int bq, int bk, int Tq, int Tk, uint8_t *__restrict__ sched,
                uint8_t *__restrict__ bm_out) {
    const ScheduleLayout lay = schedule_layout(B, H, L, bq, bk);
    const int G = lay.groups;
    const int tid = threadIdx.x;
    if (blockIdx.x < 16) {
        __shared__ int s_len[kSortMax], s_ord[kSortMax], s_tot[kSchedThreads / 64];
        const int x = blockIdx.x & 7, K = blockIdx.x < 8 ? 1 : 2;
        int4 *items = reinterpret_cast<int4 *>(sched + (K == 1 ? lay.items1 : lay.items2));
        // Batch entries by decreasing length, ties by index (rank by counting).
        const bool sorted = B <= kSortMax;
        if (sorted) {
            for (int c = tid; c < B; c += kSchedThreads) s_len[c] = clamp_len(seq_lens[c], L);
            __syncthreads();
            for (int c = tid; c < B; c += kSchedThreads) {
                const int nc = s_len[c];
                int rank = 0;
#pragma unroll 8
                for (int c2 = 0; c2 < B; ++c2) {
                    const int m = s_len[c2];
                    rank += (m > nc) || (m == nc && c2 < c);
                }
                s_ord[rank] = c;
            }
            __syncthreads();
        }
        const int pairs = B * H;
        const int npx = pairs > x ? (pairs - x + 7) / 8 : 0;  // pairs of XCD x
        const int64_t cap = ((int64_t)(pairs + 7) / 8) * G * K;  // slots of XCD x
        // Pass 0 counts the XCD's compute items (tiles with valid rows) and
        // zero items; passes 1 and 2 write them, each kind of list in pair
        // order, zero item j following compute item h + floor(j R / Nz)
        // (R = Nc - h), so compute item c >= h sits at c + ceil((c - h) Nz / R)
        // and zero item j at j + h + floor(j R / Nz) + 1.  One kind: h = Nc
        // (the zero items after the compute items) when Nz <= Nc, else h = 0
        // (spread between all of them).  Two kinds: h = floor(Nc / 2).
        // Per chunk of 256 pairs: each pair's first item and its (b, h, n), so
        // that all threads write the chunk's items together.  A thread finds
        // its item's pair in an owner map (one byte per item, when the chunk
        // has at most kOwnerMax items) or by binary search over the first
        // items.
        constexpr int kOwnerMax = 4096;
        __shared__ int s_off[kSchedThreads], s_b[kSchedThreads], s_h[kSchedThreads],
            s_n[kSchedThreads];
        __shared__ uint8_t s_owner[kOwnerMax];
        int64_t nc = 0, nz = 0;
        for (int pass = 0; pass < 3; ++pass) {
            int64_t k = 0;  // items of this list written so far
            for (int j0 = 0; j0 < npx; j0 += kSchedThreads) {
                const int j = j0 + tid;
                const bool valid = j < npx;
                const int pair = x + 8 * (valid ? j : 0);
                const int r = pair / H, h = pair - r * H;
                const int b = sorted ? s_ord[r] : r;
                const int n = sorted ? s_len[b] : clamp_len(seq_lens[b], L);
                const int real = (n + 127) / 128;
                const int zero = (G - real + kZeroTiles - 1) / kZeroTiles;
                if (pass == 0) {
                    int tc, tz;
                    block_exclusive_scan(valid ? K * real : 0, s_tot, &tc);
                    block_exclusive_scan(valid ? K * zero : 0, s_tot, &tz);
                    nc += tc;
                    nz += tz;
                    continue;
                }
                const int cnt = valid ? K * (pass == 1 ? real : zero) : 0;
                int total;
                s_off[tid] = block_exclusive_scan(cnt, s_tot, &total);
                s_b[tid] = b;
                s_h[tid] = h;
                s_n[tid] = n;
                const bool owner_map = total <= kOwnerMax;
                if (owner_map)
                    for (int i = 0; i < cnt; ++i) s_owner[s_off[tid] + i] = (uint8_t)tid;
                __syncthreads();
                const int64_t hc = K == 2 ? nc / 2 : (nz <= nc ? nc : 0), rest = nc - hc;
                for (int e = tid; e < total; e += kSchedThreads) {
                    // Without the owner map: the last pair whose first item is
                    // at or before e (pairs without items share their
                    // successor's first item).
                    int lo = 0, hi = kSchedThreads - 1;
                    if (owner_map)
                        lo = s_owner[e];
                    else
                        while (lo < hi) {
                            const int mid = (lo + hi + 1) >> 1;
                            if (s_off[mid] <= e)
                                lo = mid;
                            else
                                hi = mid - 1;
                        }
                    const int pb = s_b[lo], ph = s_h[lo], pn = s_n[lo];
                    const int preal = (pn + 127) / 128;
                    const int per = pass == 1 ? preal : (G - preal + kZeroTiles - 1) / kZeroTiles;
                    const int i = e - s_off[lo];
                    const int kind = i >= per ? 1 : 0, u = i - kind * per;
                    const int t = pass == 1 ? u : preal + kZeroTiles * u;
                    const int64_t idx = k + e;
                    int64_t pos;
                    if (pass == 1)
                        pos = idx < hc || nz == 0 ? idx
                                                  : idx + floor_div((idx - hc) * nz + rest - 1, rest);
                    else
                        pos = idx + (rest == 0 ? hc : hc + floor_div(idx * rest, nz) + 1);
                    items[8 * pos + x] = make_int4(pb, ph, t | (kind << 30), pn);
                }
                __syncthreads();  // s_off and the pair arrays are rewritten by the next chunk
                k += total;
            }
        }
        for (int64_t kk = nc + nz + tid; kk < cap; kk += kSchedThreads)
            items[8 * kk + x] = make_int4(0, 0, -1, 0);
        return;
    }

    // Entry lists: one wave per (direction, batch entry, group).
    const int lane = tid & 63;
    const int64_t idx = (int64_t)(blockIdx.x - 16) * (kSchedThreads / 64) + (tid >> 6);
    const int64_t per_dir = (int64_t)B * G;
    if (idx >= 2 * per_dir) {
        // Padding-only block mask: one wave per block row (b, i).
        const int64_t row = idx - 2 * per_dir;
        if (bm_out == nullptr || row >= (int64_t)B * Tq) return;
        const int b = (int)(row / Tq), i = (int)(row % Tq);
        const int n = clamp_len(seq_lens[b], L);
        uint8_t *out = bm_out + ((int64_t)b * Tq + i) * Tk;
        for (int j = lane; j < Tk; j += 64) out[j] = (uint8_t)padding_entry(i, j, n, bq, bk);
        return;
    }
    const int dir = (int)(idx / per_dir);
    const int b = (int)((idx % per_dir) / G), g = (int)(idx % G);
    const int n = clamp_len(seq_lens[b], L);
    const uint8_t *bmb = bm + (int64_t)b * Tq * Tk;
    uint32_t *list;
    int lines, nblk, stride;
    int64_t line_step, entry_step;
    const uint8_t *first;
    if (dir == 0) {  // query group: block rows g R .. g R + R - 1, entries along the row
        const int R = 128 / bq, line0 = g * R;
        lines = min(R, Tq - line0);
        nblk = min(Tk, (n + bk - 1) / bk);
        first = bmb + (int64_t)line0 * Tk;
        line_step = Tk;
        entry_step = 1;
        stride = lay.qstride;
        list = reinterpret_cast<uint32_t *>(sched + lay.qlists) + ((int64_t)b * G + g) * stride;
    } else {  // key group: block columns g C .. g C + C - 1, entries down the column
        const int C = 128 / bk, col0 = g * C;
        lines = min(C, Tk - col0);
        nblk = min(Tq, (n + bq - 1) / bq);
        first = bmb + col0;
        line_step = 1;
        entry_step = Tk;
        stride = lay.kstride;
        list = reinterpret_cast<uint32_t *>(sched + lay.klists) + ((int64_t)b * G + g) * stride;
    }
    int cnt = 0;
    for (int e0 = 0; e0 < nblk; e0 += 64) {
        const int e = e0 + lane;
        uint32_t kept = 0, full = 0;
        if (e < nblk) {
            for (int r = 0; r < lines; ++r) {
                uint32_t v;
                if (bm_out != nullptr)  // padding only: the closed form
                    v = dir == 0 ? padding_entry(g * (128 / bq) + r, e, n, bq, bk)
                                 : padding_entry(e, g * (128 / bk) + r, n, bq, bk);
                else
                    v = first[(int64_t)r * line_step + (int64_t)e * entry_step];
                kept |= (v != 0 ? 1u : 0u) << r;
                full |= ((v >> 1) & 1u) << r;
            }
        }
        const uint64_t m = __ballot(kept != 0);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (kept != 0) list[1 + cnt + before] = (uint32_t)e | (kept << 24) | (full << 28);
        cnt += __popcll(m);
    }
    if (lane == 0) list[0] = (uint32_t)cnt;
    for (int i = 1 + cnt + lane; i < stride; i += 64) list[i] = 0u;  // every word written
}

hipError_t launch_schedule(const int32_t *seq_lens, const uint8_t *block_mask, int B, int H,
                           int L, int block_q, int block_k, void *schedule, hipStream_t stream,
                           uint8_t *padding_mask_out) {
    const ScheduleLayout lay = schedule_layout(B, H, L, block_q, block_k);
    const int Tq = (int)(((int64_t)L + block_q - 1) / block_q);
    const int Tk = (int)(((int64_t)L + block_k - 1) / block_k);
    int64_t waves = 2 * (int64_t)B * lay.groups;
    if (padding_mask_out != nullptr) waves += (int64_t)B * Tq;
    const int64_t blocks = 16 + (waves + kSchedThreads / 64 - 1) / (kSchedThreads / 64);
    hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)blocks), dim3(kSchedThreads), 0, stream,
                       seq_lens, block_mask, B, H, L, block_q, block_k, Tq, Tk,
                       reinterpret_cast<uint8_t *>(schedule), padding_mask_out);
    return hipGetLastError();
}

}  // namespace sigattn
