// Device-side building blocks shared by the gfx950 kernels: bf16 vector
// types, the 32x32x16 bf16 MFMA, 16-byte global loads, and the key order
// used when a tile is stored transposed in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace sigattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum Bias { kBiasNone = 0, kBiasLogSeqlen = 1, kBiasLogPadlen = 2 };

// D[32x32] += A[32x16] * B[16x32], bf16 inputs, fp32 accumulation.
// Lane l holds A[l % 32][8 * (l / 32) + e] and B[8 * (l / 32) + e][l % 32]
// for e = 0..7; acc[4 * i + j] is D[8 * i + 4 * (l / 32) + j][l % 32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_len(int n, int L) { return n < 0 ? 0 : (n > L ? L : n); }

// Position of key x (0..15 inside a group of 16) in a transposed LDS row.
// The C fragment of a 32x32 MFMA gives lane half h the rows 4h..4h+3 and
// 8+4h..8+4h+3 of each 16-row group; storing the keys with bits 2 and 3
// swapped makes those 8 keys one contiguous 16-byte run, so the transposed
// operand of the next MFMA is a single 128-bit LDS read.
__device__ __forceinline__ int perm16(int x) {
    return (x & ~15) | (x & 3) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte chunks addressed by
// lanes 4 j + i / 4 (j = 0..3).  With every lane pointing at 4 consecutive
// columns of a row-major tile, the group hands each lane one column taken
// down four rows: the K-contiguous operand of an MFMA read from a tile whose
// contiguous axis is the MFMA's M or N axis.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16 *p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    bf16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return r;
}

// Raw buffer descriptors: loads beyond num_records bytes return zeros, so a
// descriptor limited to the valid rows of a sequence zero-fills padded rows
// without branches and never reads them.  Word 3 selects 32-bit data format.
constexpr int kBufferWord3 = 0x00020000;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t num_bytes) {
    const int n = num_bytes <= 0 ? 0 : (num_bytes > 0x7fffffff ? 0x7fffffff : (int)num_bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, kBufferWord3);
}

__device__ __forceinline__ uint4 buffer_load16(rsrc_t r, int byte_offset) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint8_t buffer_load_u8(rsrc_t r, int byte_offset) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, byte_offset, 0, 0);
}

// Buffer load that writes LDS instead of registers (gfx950, 16 bytes per
// lane): lane l's 16 bytes at byte_offset land at lds + 16 * l, so one wave
// instruction fills one contiguous KiB; lds must be the same in all lanes.
// Out-of-range lanes write zeros, as a register load would return them.
// Completion counts in vmcnt (wait_vm0 before a barrier that publishes it).
__device__ __forceinline__ void lds_load16(rsrc_t r, void *lds, int byte_offset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds, 16, byte_offset, 0, 0, 0);
}

// s_waitcnt vmcnt(0), leaving the other counters alone.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// What a wave stages for a tile: nothing (its block-mask line leaves the
// tile out), all-ones words (its entry is full) or the mask itself.
enum { kWantNone = 0, kWantFull = 1, kWantMask = 2 };

// Iterates, in increasing order, the tiles of BT rows that one row (or one
// column) of the block mask marks active, clipped to the n valid rows.  One
// wave ballot reads 64 block-mask entries at a time; the result is uniform,
// so the schedule lives in scalar registers.  A null block mask marks all
// entries active (padding only).  ROW: the schedule walks along block-mask
// rows (entry e of line r at bm[r * tk + e]), else down columns (at
// bm[e * tk + r]); tk is the length of a block-mask row.
// The kernel tiles along R adjacent lines of the block matrix (block rows for
// the query side, block columns for dK/dV) that one workgroup's waves share:
// a tile is visited when any line keeps it, and want() says what the calling
// wave's own line (`line`) needs of it: kWantNone when that line drops it, so
// every element still obeys its own entry.  Lines at or past `lines` are off.
// Only the union and the wave's own line are kept, in six scalar registers.
template <int BT, int R, bool ROW>
struct TileSchedule {
    const uint8_t *bm;        // line 0's first entry, or null (from seq_lens)
    int tk;                   // entries per block-mask row
    int nlines, line;         // lines that exist; the wave's own line
    int nblk;                 // block-mask entries covering [0, n)
    int per_blk;              // kernel tiles per block-mask entry
    int nkt;                  // kernel tiles covering [0, n)
    int wbase, entry, sub;
    uint64_t act;             // entries (of the 64 at wbase) some line keeps
    uint64_t mine, mine_full; // entries the wave's line keeps / marks full
    bool on, full;            // the same two, for the tile next() returned

    __device__ __forceinline__ void init(const uint8_t *first, int row_len, int lines, int own_line,
                                         int n, int block) {
        bm = first;
        tk = row_len;
        nlines = lines;
        line = own_line;
        nblk = (n + block - 1) / block;
        per_blk = block / BT;
        nkt = (n + BT - 1) / BT;
        wbase = -64;
        entry = -1;
        sub = 0;
        act = mine = mine_full = 0;
        on = full = false;
    }

    // Offset of entry e of line r from line 0's first entry.
    __device__ __forceinline__ int64_t at(int r, int e) const {
        return ROW ? (int64_t)r * tk + e : (int64_t)e * tk + r;
    }

    // Next kernel tile some line keeps, or -1.
    __device__ __forceinline__ int next() {
        if (entry >= 0 && sub + 1 < per_blk && entry * per_blk + sub + 1 < nkt) {
            ++sub;
            return entry * per_blk + sub;
        }
        while (act == 0) {
            wbase += 64;
            if (wbase >= nblk) return -1;
            const int e = wbase + (int)(threadIdx.x & 63);
            if constexpr (R == 1) {
                // One line: every visited tile is the wave's own.
                const int v = e < nblk ? (bm == nullptr ? 1 : (int)bm[at(0, e)]) : 0;
                act = __ballot(v != 0);
                mine_full = __ballot((v & 2) != 0);
            } else {
                // A rolled loop: unrolled, the lines' addresses stay live
                // across the kernel's main loop.
                mine = mine_full = 0;
                const uint8_t *pe = bm == nullptr ? nullptr : bm + at(0, e);
#pragma unroll 1
                for (int r = 0; r < nlines; ++r) {
                    const int v = e < nblk ? (pe == nullptr ? 1 : (int)*pe) : 0;
                    const uint64_t kept = __ballot(v != 0);
                    act |= kept;
                    if (r == line) {
                        mine = kept;
                        mine_full = __ballot((v & 2) != 0);
                    }
                    if (pe != nullptr) pe += ROW ? tk : 1;
                }
            }
        }
        const int bit = __builtin_ctzll(act);
        entry = wbase + bit;
        on = R == 1 || ((mine >> bit) & 1u);
        full = (mine_full >> bit) & 1u;
        act &= act - 1;
        sub = 0;
        return entry * per_blk;
    }

    // What the wave's line needs of the current tile's element mask.
    __device__ __forceinline__ int want() const {
        if constexpr (R == 1)
            return full ? kWantFull : kWantMask;
        else
            return !on ? kWantNone : full ? kWantFull : kWantMask;
    }
};

// The same walk over a kept-entry list from a schedule buffer (a count word,
// then e | kept-by-line << 24 | full-by-line << 28 per entry some line
// keeps, in increasing e): 64 list words per vector load, one read out per
// tile, and no empty entry is ever visited.  Kernels built for a schedule use
// this instead of TileSchedule, so neither carries the other's registers.
template <int BT, int R>
struct ListSchedule {
    const uint32_t *list;     // the group's list, count word first
    int cnt, cap;             // entries in the list; words after the count word
    int base, pos;            // first entry held in `words`; next entry to return
    int line;                 // the wave's own line
    int per_blk, nkt;         // kernel tiles per block-mask entry; covering [0, n)
    int entry, sub;
    uint32_t words;           // entries base .. base + 63, one per lane
    bool on, full;            // the wave's line keeps / marks full the current entry

    __device__ __forceinline__ void init(const uint32_t *lst, int lst_cap, int own_line, int n,
                                         int block) {
        const int lane = (int)(threadIdx.x & 63);
        list = lst;
        cap = lst_cap;
        cnt = (int)list[0];
        base = pos = 0;
        line = own_line;
        per_blk = block / BT;
        nkt = (n + BT - 1) / BT;
        entry = -1;
        sub = 0;
        on = full = false;
        words = lane < cap ? list[1 + lane] : 0u;
    }

    __device__ __forceinline__ int next() {
        if (entry >= 0 && sub + 1 < per_blk && entry * per_blk + sub + 1 < nkt) {
            ++sub;
            return entry * per_blk + sub;
        }
        if (pos >= cnt) return -1;
        if (pos - base >= 64) {  // the next 64 list words
            base += 64;
            const int lane = (int)(threadIdx.x & 63);
            words = base + lane < cap ? list[1 + base + lane] : 0u;
        }
        const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)words, pos - base);
        ++pos;
        entry = (int)(w & 0xffffffu);
        on = R == 1 || ((w >> (24 + line)) & 1u);
        full = (w >> (28 + line)) & 1u;
        sub = 0;
        return entry * per_blk;
    }

    __device__ __forceinline__ int want() const {
        if constexpr (R == 1)
            return full ? kWantFull : kWantMask;
        else
            return !on ? kWantNone : full ? kWantFull : kWantMask;
    }
};

// The schedule type of a kernel built with (LIST) or without a schedule.
template <int BT, int R, bool ROW, bool LIST>
using Schedule =
    typename std::conditional<LIST, ListSchedule<BT, R>, TileSchedule<BT, R, ROW>>::type;

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS
// round trips): row_shr 1, 2, 4, 8 scan each row of 16 lanes (lanes shifted
// in from outside the row add 0), then row_bcast 15 adds row 0's total to row
// 1 and row 2's to row 3, and row_bcast 31 adds the total of rows 0-1 to rows
// 2 and 3.  Lanes a move does not write keep the 0 it starts from.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Sum over each aligned group of G lanes (G = 8 or 16), every lane of a group
// receiving its group's sum, with DPP moves (no LDS round trips): swap
// neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), then mirror
// within 8 lanes (the other quad's sum) and, for 16, within the row.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
    auto mv = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                             0xf, 0xf, false));
    };
    x += mv(x, std::integral_constant<int, 0xb1>{});   // quad_perm 1,0,3,2
    x += mv(x, std::integral_constant<int, 0x4e>{});   // quad_perm 2,3,0,1
    x += mv(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
    if constexpr (G == 16) x += mv(x, std::integral_constant<int, 0x140>{});  // row_mirror
    return x;
}

// Work item of a workgroup in a launch over (batch entry, head, tile) items of
// up to two kinds: NT0 tiles of ROWS0 rows and NT1 tiles of ROWS1 rows per
// (batch entry, head) (NT1 = 0 for a launch of one kind).
//
// Placement: workgroups are dealt to the 8 XCDs round-robin by linear index
// and each XCD has its own L2, so XCD x = i % 8 owns the pairs x, x + 8, ...
// of the (length rank, head) order: all tiles of one (batch entry, head)
// share an L2, and every XCD gets one head of each batch entry when H is a
// multiple of 8.
//
// Order inside an XCD (its k-th workgroup, k = i / 8): every tile that holds
// valid rows, pair by pair from the longest sequence down (longest processing
// time first; kind 0 before kind 1 within a pair), then the tiles of empty
// sequences (n = 0), which only write zeros.  The other fully padded tiles
// get no workgroup of their own: the tiles with valid rows of the same pair
// and kind write their zeros (padded_share), so those writes overlap compute
// and hold no slot.  Workgroups past the last item return false.
//
// Computed by every wave of the workgroup alike (the result is uniform):
// lane b ranks batch entry b against all others (read back with readlane,
// ties broken by index) and pushes its length to lane rank(b), so lane r
// holds the r-th longest length; then wave prefix sums (DPP) over the XCD's
// pairs locate item k, 64 pairs at a time.  Batches of more than 64 entries
// keep their natural order.  n is the clamped length of the chosen batch
// entry.  Returns false past the last item.
template <int ROWS0, int ROWS1>
__device__ __forceinline__ bool tile_item2(const int32_t *seq_lens, int B, int H, int L, int nt0,
                                           int nt1, int &b, int &h, int &kind, int &t, int &n) {
    const int lane = (int)(threadIdx.x & 63);
    const int x = blockIdx.x & 7;
    int k = blockIdx.x >> 3;
    const int pairs = B * H;
    const int npx = pairs > x ? (pairs - x + 7) / 8 : 0;  // pairs owned by XCD x
    int sorted_b = lane, sorted_n = 0;
    if (B <= 64) {
        const int nl = lane < B ? clamp_len(seq_lens[lane], L) : -1;
        int rank = 0;
        for (int c = 0; c < B; ++c) {
            const int m = __builtin_amdgcn_readlane(nl, c);
            rank += (m > nl) || (m == nl && c < lane);
        }
        // Lanes >= B all rank B (< 64) and only overwrite an unused lane.
        sorted_b = __builtin_amdgcn_ds_permute(rank * 4, lane);
        sorted_n = __builtin_amdgcn_ds_permute(rank * 4, nl);
    }
    for (int pass = 0; pass < 2; ++pass) {  // 0: tiles with valid rows, 1: padded tiles
        for (int j0 = 0; j0 < npx; j0 += 64) {
            const int j = j0 + lane;
            const bool valid = j < npx;
            const int pair = x + 8 * (valid ? j : 0);
            const int r = pair / H;
            int bj, nj;
            if (B <= 64) {
                bj = __shfl(sorted_b, r);
                nj = __shfl(sorted_n, r);
            } else {
                bj = r;
                nj = clamp_len(seq_lens[r], L);
            }
            const int real0 = (nj + ROWS0 - 1) / ROWS0;
            const int real1 = nt1 > 0 ? (nj + ROWS1 - 1) / ROWS1 : 0;
            // Items of kind 0 in this pass; pass 1 holds only empty sequences.
            const bool empty = nj == 0;
            const int first = pass == 0 ? real0 : (empty ? nt0 : 0);
            const int cnt = valid ? first + (pass == 0 ? real1 : (empty ? nt1 : 0)) : 0;
            const int incl = wave_inclusive_scan(cnt);
            const int total = __builtin_amdgcn_readlane(incl, 63);
            if (k < total) {
                const int jl = __builtin_ctzll(__ballot(incl > k));
                const int idx = k - __builtin_amdgcn_readlane(incl - cnt, jl);
                const int f = __builtin_amdgcn_readlane(first, jl);
                h = __builtin_amdgcn_readlane(pair, jl) % H;
                b = __builtin_amdgcn_readlane(bj, jl);
                n = __builtin_amdgcn_readlane(nj, jl);
                kind = idx < f ? 0 : 1;
                t = kind == 0 ? idx : idx - f;
                return true;
            }
            k -= total;
        }
    }
    return false;
}

template <int ROWS>
__device__ __forceinline__ bool tile_item(const int32_t *seq_lens, int B, int H, int L,
                                          int ntiles, int &b, int &h, int &t, int &n) {
    int kind;
    return tile_item2<ROWS, ROWS>(seq_lens, B, H, L, ntiles, 0, b, h, kind, t, n);
}

// The workgroup's item: read from the schedule's item array in kernels built
// for a schedule (one scalar load), else derived from seq_lens (tile_item2,
// same placement and order).  Launches over 128-row tiles of one or two kinds.
template <int KINDS, bool LIST>
__device__ __forceinline__ bool work_item(const AttnParams &p, int &b, int &h, int &kind, int &t,
                                          int &n) {
    if constexpr (LIST) {
        const int4 it = (KINDS == 2 ? p.items2 : p.items1)[blockIdx.x];
        if (it.z < 0) return false;
        b = it.x;
        h = it.y;
        kind = (it.z >> 30) & 1;
        t = it.z & 0x3fffffff;
        n = it.w;
        return true;
    } else {
        const int nt = (p.L + 127) / 128;
        kind = 0;
        return tile_item2<128, 128>(p.seq_lens, p.B, p.H, p.L, nt, KINDS == 2 ? nt : 0, b, h,
                                    kind, t, n);
    }
}

// Rows a zero item (its tile starts at or past n) writes from row r0:
// kZeroTiles tiles with a schedule (its zero items cover runs of that many),
// one tile without (every tile of an empty sequence is its own item).
template <int ROWS, bool LIST>
__device__ __forceinline__ int zero_item_rows(int r0, int L) {
    return min(LIST ? kZeroTiles * ROWS : ROWS, L - r0);
}

// Without a schedule, the fully padded tiles (of ROWS rows) that tile t of a
// sequence with real = ceil(n / ROWS) tiles holding valid rows writes zeros
// for: tiles real + i with i = t, t + real, t + 2 real, ... below nt.  Calls
// f(first_row, rows) for each.  (A schedule gives these tiles zero items of
// their own.)
template <int ROWS, typename F>
__device__ __forceinline__ void padded_share(int t, int n, int L, F &&f) {
    const int real = (n + ROWS - 1) / ROWS, nt = (L + ROWS - 1) / ROWS;
    if (real == 0) return;
    for (int i = real + t; i < nt; i += real) f(i * ROWS, min(ROWS, L - i * ROWS));
}

__host__ __forceinline__ dim3 tile_grid(int ntiles, int B, int H) {
    const int64_t pairs_per_xcd = ((int64_t)B * H + 7) / 8;
    return dim3((unsigned)(8 * pairs_per_xcd * ntiles));
}

// Unpadded row-major [rows][D] bf16 tile in LDS with an XOR swizzle: the
// 16-byte chunk c of row r sits at chunk position c ^ swz(r).  swz maps any 8
// consecutive rows to 8 distinct chunk positions (16-byte reads of one
// column chunk down 8 rows hit all 32 banks), and maps the 4 rows x 2
// adjacent chunks touched by 16 lanes of a transposing read to 8 distinct
// positions as well, so both access patterns are free of bank conflicts.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
    return r * D + ((((col >> 3) ^ swz(r)) << 3) | (col & 7));
}

__device__ __forceinline__ uint4 load16(const bf16 *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 pack8(const float *x) {
    f32x2 a = {x[0], x[1]}, b = {x[2], x[3]}, c = {x[4], x[5]}, d = {x[6], x[7]};
    bf16x2 pa = __builtin_convertvector(a, bf16x2);
    bf16x2 pb = __builtin_convertvector(b, bf16x2);
    bf16x2 pc = __builtin_convertvector(c, bf16x2);
    bf16x2 pd = __builtin_convertvector(d, bf16x2);
    bf16x8 r = {pa[0], pa[1], pb[0], pb[1], pc[0], pc[1], pd[0], pd[1]};
    return r;
}

__device__ __forceinline__ bf16x4 pack4(float x0, float x1, float x2, float x3) {
    f32x2 a = {x0, x1}, b = {x2, x3};
    bf16x2 pa = __builtin_convertvector(a, bf16x2);
    bf16x2 pb = __builtin_convertvector(b, bf16x2);
    bf16x4 r = {pa[0], pa[1], pb[0], pb[1]};
    return r;
}

// Sigmoid weight of one score.  The MFMA operand held in registers was
// scaled by -scale * log2(e) beforehand (scale8), so the accumulator is
// already u = -scale * (q . k) * log2(e), and with C = exp(-b):
//   sigma(scale * (q . k) + b) = 1 / (1 + C * 2^u).
// 2^u overflowing to +inf gives 0 and underflowing to 0 gives 1, the limits.
__device__ __forceinline__ float sigmoid_scaled(float u, float cexp) {
    return __builtin_amdgcn_rcpf(fmaf(__builtin_amdgcn_exp2f(u), cexp, 1.0f));
}

// Eight bf16 values times s, rounded back to bf16 (once per workgroup on the
// operand held in registers: it folds the score scale into the dot product).
__device__ __forceinline__ bf16x8 scale8(bf16x8 x, float s) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)x[e] * s;
    return pack8(f);
}

// Branch-free select: x where keep, else 0 (a bit mask, so the compiler does
// not turn the choice into control flow around the work that produced x).
__device__ __forceinline__ float keep_or_zero(float x, bool keep) {
    return __uint_as_float(__float_as_uint(x) & (keep ? 0xffffffffu : 0u));
}

// x where `keep` is all ones, -inf where it is zero (one bitfield insert).
__device__ __forceinline__ float keep_bits_or_neg_inf(float x, uint32_t keep) {
    return __uint_as_float((__float_as_uint(x) & keep) | (0xff800000u & ~keep));
}

// A score accumulator where `keep` is all ones, else the value whose weight is
// exactly 0: -inf for a softmax logit (2^-inf = 0), +inf for a sigmoid
// exponent u (1 / (1 + C 2^u) = 1 / inf = 0).
template <bool SOFT>
__device__ __forceinline__ float keep_score(float x, uint32_t keep) {
    constexpr uint32_t kDrop = SOFT ? 0xff800000u : 0x7f800000u;
    return __uint_as_float((__float_as_uint(x) & keep) | (kDrop & ~keep));
}

__device__ __forceinline__ float bias_value(int mode, int n, int L) {
    if (mode == kBiasLogSeqlen) return -logf((float)n);
    if (mode == kBiasLogPadlen) return -logf((float)L);
    return 0.0f;
}

// exp(-b) for the bias modes above: n, L or 1, exactly.
__device__ __forceinline__ float bias_factor(int mode, int n, int L) {
    if (mode == kBiasLogSeqlen) return (float)n;
    if (mode == kBiasLogPadlen) return (float)L;
    return 1.0f;
}

// ---------------------------------------------------------------------------
// Element mask of one tile as bits.  Inside a tile that the binary block mask
// keeps, the element mask still decides every (query, key) entry (Binary Block
// Masking, "How it works").  Gathering those bytes lane by lane in the MFMA
// layout costs one cache line per lane per byte; instead a workgroup reads the
// tile's mask rows with coalesced 16-byte loads, one 32-key word per thread,
// and leaves a bit per entry in LDS.
//
// Word (wi, r) of a tile with mask rows [r0, r0 + ROWS) and keys
// [k0, k0 + KEYS) holds keys k0 + 32 wi + t of row r0 + r at bit
// 8 (t % 4) + t / 4: the order in which a per-dword non-zero test of the 32
// mask bytes delivers them.  Rows and keys at or past n are 0.  LDS layout:
// words[wi * ROWS + r].  Mask rows are L bytes long and not aligned; the
// 16-byte loads do not need to be.
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    return (((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;  // bit 7 of each byte
}

// Bit of key t (0..31) within a word.
__device__ __forceinline__ constexpr int mask_bit(int t) { return 8 * (t & 3) + (t >> 2); }

// All-ones (keep) or zero (drop) from bit `pos` of word.
__device__ __forceinline__ uint32_t mask_select(uint32_t word, int pos) {
    return (uint32_t)__builtin_amdgcn_sbfe((int)word, pos, 1);
}

// Element-mask kinds of the attention kernels: none, dense bytes [L, L] per
// batch entry, one key range [lo, hi] per query row (causal, packed
// documents, sliding windows: the masks whose rows are intervals), or the
// dense mask packed to bits by the block-mask builder (in a schedule).
enum { kMaskNone = 0, kMaskDense = 1, kMaskRange = 2, kMaskBits = 3 };

// One batch entry's element mask, in the form the kernel was built for.
struct MaskSource {
    rsrc_t bytes;          // dense: exactly its L x L bytes
    const int32_t *range;  // ranges: [L, 2] (lo, hi) per query row
    const uint32_t *bits;  // packed: [L, W] words, bit t of word w = key 32 w + t
    int L, W;
};

// Where key t (0..31) of a mask word sits: dense words keep the order in
// which the byte test delivers them, range words the natural order.
template <int MASK>
__device__ __forceinline__ constexpr int key_bit(int t) {
    return MASK == kMaskDense ? mask_bit(t) : t;
}

// What a wave's share of a masked tile needs, from the OR and the AND of the
// mask words its lanes hold: kSkip (no entry kept: no work at all), kDense
// (every entry kept) or kMixed.
enum { kSkip = 0, kDense = 1, kMixed = 2 };
__device__ __forceinline__ int mask_class(uint32_t any_bits, uint32_t all_bits) {
    if (__ballot(any_bits != 0u) == 0) return kSkip;
    if (__ballot(all_bits != 0xffffffffu) == 0) return kDense;
    return kMixed;
}

template <int ROWS, int KEYS, int NT, bool WAVE_ROWS>
struct MaskStage {
    // Wave w stages the words it reads itself: with WAVE_ROWS, every word of
    // rows 32 w .. 32 w + 31 (the waves split the query rows); otherwise word
    // w of all 32 rows (the waves split the keys).  So the wave learns what
    // its next tile needs (mask_class) while it stages it.
    static constexpr int kWordsPerRow = KEYS / 32;
    static constexpr int kWords = ROWS * kWordsPerRow;
    static constexpr int kWordsPerWave = WAVE_ROWS ? kWordsPerRow : 1;
    static_assert(kWordsPerWave <= 2, "at most one word per lane");
    static_assert(WAVE_ROWS ? ROWS == NT / 2 : (ROWS == 32 && kWordsPerRow == NT / 64),
                  "one wave per 32 rows, or per 32 keys");
    uint4 lo, hi;
    int r, wi;
    bool act;

    __device__ __forceinline__ void init(int tid) {
        const int lane = tid & 63, w = tid >> 6;
        r = (WAVE_ROWS ? 32 * w : 0) + (lane & 31);
        wi = (WAVE_ROWS ? 0 : w) + (lane >> 5);
        act = (lane >> 5) < kWordsPerWave;
    }

    // src.bytes covers exactly the batch entry's L x L mask; L * L fits in
    // int.  Words of rows or keys at or past n are not read (store clears
    // them), nor any word of a full tile (every entry valid: store writes ones).
    __device__ __forceinline__ void load(const MaskSource &src, int n, int r0, int k0, int want) {
        lo = hi = make_uint4(0u, 0u, 0u, 0u);
        const int row = r0 + r, key = k0 + 32 * wi, L = src.L;
        if (want != kWantMask || !act || row >= n || key >= n) return;
        const int off = row * L + key;
        if (off + 32 <= L * L) {
            lo = buffer_load16(src.bytes, off);
            hi = buffer_load16(src.bytes, off + 16);
        } else {
            // The last row's window runs past the end of the mask, where the
            // range check would drop a 16-byte load whole: byte by byte, the
            // bytes past the end reading 0.
            uint32_t x[8] = {};
#pragma unroll
            for (int t = 0; t < 32; ++t)
                x[t >> 2] |= (uint32_t)buffer_load_u8(src.bytes, off + t) << (8 * (t & 3));
            lo = make_uint4(x[0], x[1], x[2], x[3]);
            hi = make_uint4(x[4], x[5], x[6], x[7]);
        }
    }

    // Writes the bits and returns this wave's class for the tile (all lanes
    // of the wave call it).
    __device__ __forceinline__ int store(uint32_t *words, int r0, int k0, int n, int want) const {
        if (want == kWantNone) return kSkip;  // the wave leaves this tile out
        if (want == kWantFull) {
            if (act) words[wi * ROWS + r] = 0xffffffffu;
            return kDense;
        }
        uint32_t x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if (k0 + KEYS > n) {  // keys at or past n: clear their bytes
            const int m = n - k0 - 32 * wi;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int keep = min(max(m - 4 * j, 0), 4);
                x[j] &= keep >= 4 ? 0xffffffffu : (1u << (8 * keep)) - 1u;
            }
        }
        uint32_t bits = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) bits |= nonzero_bytes(x[j]) >> (7 - j);
        if (r0 + r >= n) bits = 0u;
        if (act) words[wi * ROWS + r] = bits;
        return mask_class(bits, act ? bits : 0xffffffffu);
    }
};

// The same tile words from key ranges: the kept keys of a row are the run
// [max(lo, 0), min(hi, n - 1)], so a word is one shifted run of ones (natural
// key order) and the mask itself is never read.  Same thread mapping and
// LDS layout as MaskStage.
template <int ROWS, int KEYS, int NT, bool WAVE_ROWS>
struct RangeStage {
    static constexpr int kWordsPerRow = KEYS / 32;
    static constexpr int kWords = ROWS * kWordsPerRow;
    static constexpr int kWordsPerWave = WAVE_ROWS ? kWordsPerRow : 1;
    static_assert(kWordsPerWave <= 2, "at most one word per lane");
    static_assert(WAVE_ROWS ? ROWS == NT / 2 : (ROWS == 32 && kWordsPerRow == NT / 64),
                  "one wave per 32 rows, or per 32 keys");
    int lo, hi;  // this lane's row keeps keys [lo, hi] (empty when lo > hi)
    int r, wi;
    bool act;

    __device__ __forceinline__ void init(int tid) {
        const int lane = tid & 63, w = tid >> 6;
        r = (WAVE_ROWS ? 32 * w : 0) + (lane & 31);
        wi = (WAVE_ROWS ? 0 : w) + (lane >> 5);
        act = (lane >> 5) < kWordsPerWave;
    }

    __device__ __forceinline__ void load(const MaskSource &src, int n, int r0, int k0, int want) {
        lo = 1;
        hi = 0;
        const int row = r0 + r;
        if (want != kWantMask || !act || row >= n) return;
        const int2 kr = *reinterpret_cast<const int2 *>(src.range + 2 * row);
        lo = max(kr.x, 0);
        hi = min(kr.y, n - 1);
    }

    __device__ __forceinline__ int store(uint32_t *words, int r0, int k0, int n, int want) const {
        if (want == kWantNone) return kSkip;  // the wave leaves this tile out
        if (want == kWantFull) {
            if (act) words[wi * ROWS + r] = 0xffffffffu;
            return kDense;
        }
        const int base = k0 + 32 * wi;
        const int a = max(lo, base), e = min(hi, base + 31);
        const uint32_t bits = a > e ? 0u : ((2u << (e - a)) - 1u) << (a - base);
        if (act) words[wi * ROWS + r] = bits;
        return mask_class(bits, act ? bits : 0xffffffffu);
    }
};

// The same tile words from the packed mask: one dword load per word, already
// in natural key order.  Words of rows or keys at or past n are not read, and
// a word's bits for keys at or past n are cleared.  Same thread mapping and
// LDS layout as MaskStage.
template <int ROWS, int KEYS, int NT, bool WAVE_ROWS>
struct BitsStage {
    static constexpr int kWordsPerRow = KEYS / 32;
    static constexpr int kWords = ROWS * kWordsPerRow;
    static constexpr int kWordsPerWave = WAVE_ROWS ? kWordsPerRow : 1;
    static_assert(kWordsPerWave <= 2, "at most one word per lane");
    static_assert(WAVE_ROWS ? ROWS == NT / 2 : (ROWS == 32 && kWordsPerRow == NT / 64),
                  "one wave per 32 rows, or per 32 keys");
    uint32_t word;
    int r, wi;
    bool act;

    __device__ __forceinline__ void init(int tid) {
        const int lane = tid & 63, w = tid >> 6;
        r = (WAVE_ROWS ? 32 * w : 0) + (lane & 31);
        wi = (WAVE_ROWS ? 0 : w) + (lane >> 5);
        act = (lane >> 5) < kWordsPerWave;
    }

    __device__ __forceinline__ void load(const MaskSource &src, int n, int r0, int k0, int want) {
        word = 0u;
        const int row = r0 + r, key = k0 + 32 * wi;
        if (want != kWantMask || !act || row >= n || key >= n) return;
        word = src.bits[(int64_t)row * src.W + (key >> 5)];
    }

    __device__ __forceinline__ int store(uint32_t *words, int r0, int k0, int n, int want) const {
        if (want == kWantNone) return kSkip;  // the wave leaves this tile out
        if (want == kWantFull) {
            if (act) words[wi * ROWS + r] = 0xffffffffu;
            return kDense;
        }
        uint32_t bits = word;
        const int m = n - (k0 + 32 * wi);  // keys of this word below n
        if (m < 32) bits &= m <= 0 ? 0u : (1u << m) - 1u;
        if (r0 + r >= n) bits = 0u;
        if (act) words[wi * ROWS + r] = bits;
        return mask_class(bits, act ? bits : 0xffffffffu);
    }
};

// The stager of a mask kind (none stages nothing; MaskStage is a placeholder).
template <int MASK, int ROWS, int KEYS, int NT, bool WAVE_ROWS>
using MaskStager = typename std::conditional<
    MASK == kMaskRange, RangeStage<ROWS, KEYS, NT, WAVE_ROWS>,
    typename std::conditional<MASK == kMaskBits, BitsStage<ROWS, KEYS, NT, WAVE_ROWS>,
                              MaskStage<ROWS, KEYS, NT, WAVE_ROWS>>::type>::type;

// The batch entry's mask source of a kernel of kind MASK.
template <int MASK>
__device__ __forceinline__ MaskSource mask_source(const AttnParams &p, int b) {
    const uint8_t *mask = p.mask;
    const int32_t *key_range = p.key_range;
    const int L = p.L;
    MaskSource m;
    m.bytes = make_rsrc(MASK == kMaskDense ? mask + (int64_t)b * L * L : nullptr,
                        MASK == kMaskDense ? (int64_t)L * L : 0);
    m.range = MASK == kMaskRange ? key_range + (int64_t)b * L * 2 : nullptr;
    m.bits = MASK == kMaskBits ? p.mask_bits + (int64_t)b * L * p.bits_w : nullptr;
    m.L = L;
    m.W = p.bits_w;
    return m;
}

}  // namespace sigattn
