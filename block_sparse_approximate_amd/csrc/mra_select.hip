// mra_select.hip — step 1 low-resolution logits and step 2 block selection
// ([MRA] "第一步" and "第二步").
//
// logits_kernel: workgroup (bh, t) computes the logits of 16 block rows of
// head bh,  S_ij = fma-chain_c(qhat_i[c], khat_j[c]) * tau  (fp32, channels in
// order from +0, the canonical order), the row maximum over non-empty key
// blocks, the selection score of each cell, its ordered 32-bit key, and a
// 4096-bin histogram of the top 12 key bits, which it adds into the head's
// histogram.  In full mode it also sums the low-resolution attention of its
// rows over every key block ("第四步"), selected or not.  All workgroups of a head run on one XCD, so the head's khat is
// fetched from memory once and then served by that XCD's L2.
//
// select_kernel: one workgroup of 1024 threads per head selects the top-K
// cells:
//   * the composite key of a cell is (ordered fp32 score, then the inverse
//     flat index), so all keys differ and "the first K cells in (score
//     descending, flat index ascending)" are exactly the K largest keys;
//   * a radix select walks the key from the top: the histogram fixes the
//     first 12 bits, further 12-bit passes run only while that bin holds
//     more than kCap cells; one pass then marks the cells above the bin as
//     selected and copies the cells inside it into LDS, where 8-bit passes
//     over those candidates find the K-th largest key T;
//   * the selected set {key >= T} is written as a bitmap, as CSR (row_ptr,
//     col ascending) and as the attention stream: one record per selected
//     block, rows longer than p.seg_whole blocks cut into segments of p.chunk.
// A thread holds 16 cell keys in registers (the whole head up to N = 4096;
// longer heads are walked in tiles of 16384 cells with the next tile in
// flight), and wave w's cells of a tile are 64 consecutive cells, so one
// ballot is 64 consecutive bits of the selection.
//
// lgsel_kernel: for heads of 64 or 128 block rows (N = 2048, 4096), when
// all of its logits workgroups fit the device at once (fused_select), the
// logits and the selection run in one launch: the head's workgroups form 16
// block rows of logits each, add one to the head's arrival count, and the
// first nb / 32 of them wait for the count and select 32 rows each
// (select_rows; see the comment above lgsel_kernel).  Otherwise the
// separate logits_kernel and select_kernel launches below run.
//
// premark_kernel: for heads longer than one tile (with nb a multiple of 64)
// the marking pass runs before the selector, one workgroup per tile, so the
// selector only loads the bitmap of sure cells and the candidate list.
// Apart from lgsel_kernel's per-head count, the kernels are separate
// launches: the kernel boundary is what makes one workgroup's output visible
// to another, with no device-wide fences.
// The translation unit is built with -ffp-contract=off so that every fp32
// operation is the one written.
#include "mra_pool_unit.h"

namespace mra {
namespace {

// logits kernel shape
constexpr int kLgThreads = 512;
constexpr int kLgWaves = kLgThreads / 64;
constexpr int kRT = 2 * kLgWaves;   // block rows per logits workgroup (two per wave)
constexpr int kCT = 128;            // key blocks per logits tile

// select kernel shape
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kCells = 16;                         // cell keys per thread and tile
constexpr int kTileCells = kSelThreads * kCells;   // 16384
constexpr int kCap = kSelCap;                      // selection candidates held in LDS
constexpr int kDigitBits = 8;                      // radix digit over the candidates
constexpr int kDigitBins = 1 << kDigitBits;
constexpr int kRankSet = 64;                       // candidates few enough to be ranked pairwise

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// ---------------------------------------------------------------- LDS plans
struct LogitsLds {
    size_t qS, kS, hist, total;
};

constexpr int kMaxColTiles = 4;   // column tiles of kCT key blocks (N <= 16384)
// floats per staged qhat / khat / vhat row of a head of hd channels (4 floats
// of pad: lane l's 16-byte reads of row l spread over the banks)
__host__ __device__ constexpr int hat_stride(int hd) { return hd + 4; }
                                  // fall on banks 4l .. 4l + 3, distinct over each 16-lane phase


__host__ __device__ inline LogitsLds logits_lds(int nb, int hd) {
    LogitsLds L;
    size_t o = 0;
    L.qS = o; o = align16(o + (size_t)kRT * hat_stride(hd) * 4);   // qhat rows of the workgroup
    L.kS = o; o = align16(o + (size_t)kCT * hat_stride(hd) * 4);   // khat rows of one column tile
    L.hist = o; o = align16(o + kHistBins * 4);
    L.total = o;
    return L;
}

struct SelectLds {
    size_t hist, dig, cand, bitmap, rc, ic, mbv, scan, small, total;
};

// Heads of more than one tile of cells, with whole 64-cell groups per block
// row, get their marking pass from premark_kernel.
__host__ __device__ inline bool premarked(int nb) {
    return (nb & 63) == 0 && (size_t)nb * nb > (size_t)kTileCells;
}

__host__ __device__ inline SelectLds select_lds(int nb) {
    SelectLds L;
    const int words = (nb + 31) / 32;
    size_t o = 0;
    L.hist = o; o = align16(o + kHistBins * 4);
    L.dig = o; o = align16(o + 2 * kDigitBins * 4);
    L.cand = o; o = align16(o + (size_t)kCap * 8);
    L.bitmap = o; o = align16(o + (size_t)nb * words * 4);
    L.rc = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.ic = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.mbv = o; o = align16(o + (size_t)nb * 4);
    L.scan = o; o = align16(o + (kSelWaves + 1) * 8);
    L.small = o; o = align16(o + 32 * 4);
    L.total = o;
    return L;
}

// Heads of one tile whose block rows hold whole 64-cell groups (nb = 64 or
// 128) are selected by kTileRows-row workgroups (select_rows below).
constexpr int kTileRows = 32;
__host__ __device__ inline bool row_tiled(int nb) { return nb == 64 || nb == 128; }

struct TileLds {
    size_t hist, dig, cand, bitmap, rc, ic, mbv, wcnt, few, rank, small, total;
};

__host__ __device__ inline TileLds tile_lds(int nb) {
    TileLds L;
    const int words = (nb + 31) / 32;
    size_t o = 0;
    L.hist = o; o = align16(o + kHistBins * 4);
    L.dig = o; o = align16(o + 2 * kDigitBins * 4);
    L.cand = o; o = align16(o + (size_t)kCap * 8);
    L.bitmap = o; o = align16(o + (size_t)kTileRows * words * 4);   // the workgroup's own rows
    L.rc = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.ic = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.mbv = o; o = align16(o + (size_t)nb * 4);
    L.wcnt = o; o = align16(o + (size_t)kCells * kSelWaves * 4);
    L.few = o; o = align16(o + 64 * 8);
    L.rank = o; o = align16(o + 64 * 4);
    L.small = o; o = align16(o + 32 * 4);
    L.total = o;
    return L;
}

// ---------------------------------------------------------------- helpers
// Inclusive scan over the 64 lanes of a wave by DPP: shifts within rows of
// 16 lanes, then each row's total broadcast to the rows after it.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// The same for 64-bit values whose 32-bit halves never carry into each other
// (packed counts): each half is scanned on its own.
__device__ __forceinline__ uint64_t wave_scan_incl(uint64_t x) {
    const uint32_t lo = wave_scan_incl((uint32_t)x), hi = wave_scan_incl((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Lane E of `old` takes the wave-uniform value v (v_writelane_b32).  The
// compiler does not look into the asm for hazards, so it waits itself: five
// wait states cover an SGPR or EXEC written by the VALU just before (two and
// four needed) and a previous write of `old` by v_writelane.
template <int E>
__device__ __forceinline__ uint32_t write_lane(uint32_t old, uint32_t v) {
    asm("s_nop 4\n\tv_writelane_b32 %0, %1, %2" : "+v"(old) : "s"(v), "n"(E));
    return old;
}

// f(IntC<E>{}) for E = B .. N - 1, each E a compile-time constant.
template <int V>
struct IntC {
    static constexpr int value = V;
};
template <int B, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < N) {
        f(IntC<B>{});
        static_for<B + 1, N>(f);
    }
}

// Max and sum over the 64 lanes of a wave by DPP (the result in every lane).
// The max is exact in any order; the sum's order is fixed by the lane layout.
__device__ __forceinline__ float wave_max(float x) {
    const int ninf = __builtin_bit_cast(int, -__builtin_inff());
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x112, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x114, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x118, 0xF, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false)));
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false)));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ __forceinline__ float wave_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Exclusive scan of one value per thread over the select workgroup.
// Returns the exclusive prefix; *total gets the sum.  Uses scan[kSelWaves + 1].
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* scan, T* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T x = wave_scan_incl(v);
    if (lane == 63) scan[wave] = x;
    __syncthreads();
    if (threadIdx.x < 64) {
        const T t = threadIdx.x < kSelWaves ? scan[threadIdx.x] : T(0);
        const T y = wave_scan_incl(t);
        if (threadIdx.x < kSelWaves) scan[threadIdx.x] = y - t;
        if (threadIdx.x == kSelWaves - 1) scan[kSelWaves] = y;
    }
    __syncthreads();
    const T ex = scan[wave] + x - v;
    *total = scan[kSelWaves];
    __syncthreads();
    return ex;
}

struct BinPick {
    uint32_t bin, above, count;
};

// In a histogram of kHistBins bins held in LDS, find the bin where the count
// taken from the top first reaches `need`.  Each thread owns 4 bins; the
// whole workgroup calls this.
__device__ __forceinline__ BinPick pick_bin(const uint32_t* h, uint32_t need, uint32_t* scan, uint32_t* small) {
    constexpr int kPer = kHistBins / kSelThreads;
    const int rt = kSelThreads - 1 - (int)threadIdx.x;   // reversed: the top bins come first
    uint32_t c[kPer], local = 0;
#pragma unroll
    for (int e = 0; e < kPer; e++) {
        c[e] = h[rt * kPer + e];
        local += c[e];
    }
    uint32_t tot;
    const uint32_t above = block_excl_scan<uint32_t>(local, scan, &tot);
    if (above < need && need <= above + local) {
        uint32_t acc = above;
#pragma unroll
        for (int e = kPer - 1; e >= 0; e--) {
            if (acc < need && acc + c[e] >= need) {
                small[0] = (uint32_t)(rt * kPer + e);
                small[1] = acc;
                small[2] = c[e];
            }
            acc += c[e];
        }
    }
    __syncthreads();
    BinPick r{small[0], small[1], small[2]};
    __syncthreads();
    return r;
}

// The same over kDigitBins bins, by wave 0 alone (4 bins per lane); the
// result goes to small[0..2] for the whole workgroup to read after a barrier.
__device__ __forceinline__ void pick_digit_wave(const uint32_t* h, uint32_t need, uint32_t* small) {
    constexpr int kPer = kDigitBins / 64;
    const int lane = threadIdx.x;
    const int rt = 63 - lane;
    uint32_t c[kPer], local = 0;
#pragma unroll
    for (int e = 0; e < kPer; e++) {
        c[e] = h[rt * kPer + e];
        local += c[e];
    }
    const uint32_t above = wave_scan_incl(local) - local;
    if (above < need && need <= above + local) {
        uint32_t acc = above;
#pragma unroll
        for (int e = kPer - 1; e >= 0; e--) {
            if (acc < need && acc + c[e] >= need) {
                small[0] = (uint32_t)(rt * kPer + e);
                small[1] = acc;
                small[2] = c[e];
            }
            acc += c[e];
        }
    }
}

// Cell keys of the tile at `base` into registers, every load issued at once;
// register e holds cell base + threadIdx.x + e * kSelThreads.
__device__ __forceinline__ void fetch_keys(const uint32_t* __restrict__ G, uint32_t base, uint32_t ncell,
                                           uint32_t (&kv)[kCells]) {
    if (base + kTileCells <= ncell) {   // a full tile: no per-cell guard
#pragma unroll
        for (int e = 0; e < kCells; e++) kv[e] = G[base + threadIdx.x + e * kSelThreads];
    } else {
#pragma unroll
        for (int e = 0; e < kCells; e++) {
            const uint32_t x = base + threadIdx.x + e * kSelThreads;
            kv[e] = x < ncell ? G[x] : 0u;
        }
    }
}

// Block row of flat cell x: x / nb by a multiply-high with one correction
// step each way (x < 2^18 and nb <= 512 here).
__device__ __forceinline__ uint32_t row_of(uint32_t x, uint32_t nb, uint32_t magic) {
    uint32_t i = __umulhi(x, magic);
    if (i * nb > x) i--;
    if ((i + 1) * nb <= x) i++;
    return i;
}

// The marking pass of the selector over every cell of a head, tile by tile:
// a cell whose key prefix (the top pbits bits of the composite key) is above
// `prefix` is selected for sure and goes into the bitmap; a cell whose prefix
// equals it is a candidate and goes into the LDS list (one LDS atomic per wave
// and four 64-cell groups).  kRows64: a block row holds a multiple of 64
// cells, so a wave's 64 consecutive cells are two whole bitmap words and are
// stored without atomics.  kNarrow: pbits <= 32, so the prefix is a prefix of
// the 32-bit score key alone.
template <bool kRows64, bool kNarrow>
__device__ __forceinline__ void mark_cells(const uint32_t* __restrict__ G, uint32_t ncell, int ntiles, int nb,
                                           int words, uint32_t magic, uint64_t prefix, int pbits,
                                           uint32_t (&kv)[kCells], uint32_t* bitmap, uint64_t* cand,
                                           uint32_t* small) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)threadIdx.x - lane);
    const uint32_t sh = kNarrow ? (uint32_t)(32 - pbits) : 0u;
    const uint32_t p32 = (uint32_t)prefix;
    for (int t = 0; t < ntiles; t++) {
        const uint32_t base = (uint32_t)t * kTileCells;
        uint32_t kn[kCells];
        if (t + 1 < ntiles) fetch_keys(G, base + kTileCells, ncell, kn);   // next tile in flight
#pragma unroll
        for (int e0 = 0; e0 < kCells; e0 += 4) {
            uint64_t mh[4];
            bool hit[4];
            uint32_t tot = 0;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int e = e0 + q;
                const uint32_t x0 = base + wbase + (uint32_t)e * kSelThreads;   // the wave's first cell
                const uint32_t x = x0 + lane;
                const bool in = x < ncell;
                bool sure;
                if constexpr (kNarrow) {
                    const uint32_t top = kv[e] >> sh;
                    sure = in && top > p32;
                    hit[q] = in && top == p32;
                } else {
                    const uint64_t top = cell_key64(kv[e], x) >> (64 - pbits);
                    sure = in && top > prefix;
                    hit[q] = in && top == prefix;
                }
                const uint64_t ms = __ballot(sure);
                if constexpr (kRows64) {
                    if (x0 < ncell) {
                        const uint32_t i0 = row_of(x0, (uint32_t)nb, magic), j0 = x0 - i0 * (uint32_t)nb;
                        if (lane == 0)
                            *reinterpret_cast<uint2*>(bitmap + i0 * words + (j0 >> 5)) =
                                make_uint2((uint32_t)ms, (uint32_t)(ms >> 32));
                    }
                } else if (sure) {
                    const uint32_t i = row_of(x, (uint32_t)nb, magic), j = x - i * (uint32_t)nb;
                    atomicOr(&bitmap[i * words + (j >> 5)], 1u << (j & 31));
                }
                mh[q] = __ballot(hit[q]);
                tot += (uint32_t)__popcll(mh[q]);
            }
            if (tot) {
                uint32_t at0 = 0;
                if (lane == 0) at0 = atomicAdd(&small[8], tot);
                at0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)at0);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    if (hit[q]) {
                        const uint32_t x = base + wbase + (uint32_t)(e0 + q) * kSelThreads + lane;
                        const uint32_t at = at0 + (uint32_t)__popcll(mh[q] & lt_mask);
                        if (at < (uint32_t)kCap) cand[at] = cell_key64(kv[e0 + q], x);
                    }
                    at0 += (uint32_t)__popcll(mh[q]);
                }
            }
        }
        if (t + 1 < ntiles) {
#pragma unroll
            for (int e = 0; e < kCells; e++) kv[e] = kn[e];
        }
    }
}

// The khat tile of key blocks j0 .. j0 + kCT - 1 into registers: float4 x is
// block j0 + x / (HD / 4), channels 4 * (x % (HD / 4)) .. +3 (HD / 4 lanes
// read one row).
template <int HD>
__device__ __forceinline__ void fetch_khat(const float* __restrict__ kh, int j0, int nb,
                                           float4 (&kv)[kCT * (HD / 4) / kLgThreads]) {
#pragma unroll
    for (int e = 0; e < kCT * (HD / 4) / kLgThreads; e++) {
        const int x = threadIdx.x + e * kLgThreads, jj = x / (HD / 4), c4 = (x % (HD / 4)) * 4;
        kv[e] = j0 + jj < nb ? *reinterpret_cast<const float4*>(kh + (size_t)(j0 + jj) * HD + c4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}


// The marking pass for the common shape: one tile (kv holds every cell), a
// multiple of 64 cells per block row, every cell of the tile present, and a
// prefix of at most 32 bits.  Straight-line per 64-cell group: one shift,
// two compares (their lane masks are the ballots) and one bitmap store; the
// wave's candidates then take their place in the list with one LDS atomic
// (with many boundary cells, an atomic per group serialised the waves).
__device__ __forceinline__ void mark_cells_fast(int nb, int words, uint32_t magic, uint32_t p32, int pbits,
                                                const uint32_t (&kv)[kCells], uint32_t* bitmap, uint64_t* cand,
                                                uint32_t* small) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)threadIdx.x - lane);
    const uint32_t sh = (uint32_t)(32 - pbits);
    // sure cells straight into the bitmap; the wave's boundary cells are
    // counted first and take their place in the list with one atomic
    uint64_t mh[kCells];
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < kCells; e++) {
        const uint32_t x0 = wbase + (uint32_t)e * kSelThreads;   // the wave's first cell (uniform)
        const uint32_t top = kv[e] >> sh;
        const uint64_t ms = __ballot(top > p32);
        mh[e] = __ballot(top == p32);
        tot += (uint32_t)__popcll(mh[e]);
        const uint32_t i0 = row_of(x0, (uint32_t)nb, magic), j0 = x0 - i0 * (uint32_t)nb;
        if (lane == 0)
            *reinterpret_cast<uint2*>(bitmap + i0 * words + (j0 >> 5)) = make_uint2((uint32_t)ms, (uint32_t)(ms >> 32));
    }
    if (tot) {
        uint32_t at0 = 0;
        if (lane == 0) at0 = atomicAdd(&small[8], tot);
        at0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)at0);
#pragma unroll
        for (int e = 0; e < kCells; e++) {
            if ((mh[e] >> lane) & 1ull) {
                const uint32_t at = at0 + (uint32_t)__popcll(mh[e] & lt_mask);
                if (at < (uint32_t)kCap) cand[at] = cell_key64(kv[e], wbase + (uint32_t)e * kSelThreads + lane);
            }
            at0 += (uint32_t)__popcll(mh[e]);
        }
    }
}

// ---------------------------------------------------------------- V pooling
// Full mode's V is needed first by the low-res sums in the selector launch,
// so where the logits workgroups leave CUs free (at most one of them per
// CU) the logits launch pools V with extra workgroups (g counts them from
// 0): kVUnitsPerGroup units per workgroup, thread tid in unit tid /
// kVUnitStride; workgroup g runs on XCD g % 8 with the head's other stages.
__host__ __device__ inline int v_groups_per_head(int nb, int dt, int hd) {
    const int units = (nb + v_unit_blocks(dt, hd) - 1) / v_unit_blocks(dt, hd);
    return (units + kVUnitsPerGroup - 1) / kVUnitsPerGroup;
}

template <int DT, int HD>
__device__ __forceinline__ void pool_v(const Params& p, int g, unsigned char* smem) {
    constexpr int kUB = v_unit_blocks(DT, HD);
    const int per_head = v_groups_per_head(p.nb, DT, HD);
    const int xcd = g & 7, slot = g >> 3;
    const int hm = slot / per_head;
    const int bh = xcd + 8 * hm;
    const int unit = (slot - hm * per_head) * kVUnitsPerGroup + (int)threadIdx.x / kVUnitStride;
    const int blk0 = unit * kUB;
    pool_unit<DT, HD, kUB>(p, 2, bh, blk0, bh < p.BH && blk0 < p.nb, (int)threadIdx.x % kVUnitStride,
                           smem + (size_t)((int)threadIdx.x / kVUnitStride) * kVUnitBytes);
}

// ---------------------------------------------------------------- logits
// Wave w owns block rows ra = row0 + 2w and rb = ra + 1 of the workgroup's 16;
// lane l owns key blocks 128 t + l and 128 t + 64 + l of every column tile
// t, so the row max, the score and the key of a cell never leave the
// registers of the lane that computed its logit.  The qhat rows and the khat
// tile sit in LDS row-major; a lane reads 4 channels of each of its two key
// blocks and of the two rows at once and does the 16 fmas they feed, each
// cell's chain still going over the channels in order.
// kGiven: the logits are already in p.logits (selector hook); skip their
// computation and only form row maxima, keys and the histogram.
template <bool kGiven, int HD>
__global__ __launch_bounds__(kLgThreads) void logits_kernel(Params p) {
    constexpr int kHatStride = hat_stride(HD);
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb;
    const int tiles_per_head = (nb + kRT - 1) / kRT;
    const int n_lg = 8 * ((p.BH + 7) / 8) * tiles_per_head;   // logits workgroups; V pooling after them
    if (!kGiven && (int)blockIdx.x >= n_lg) {
        if (p.dtype == 1) pool_v<1, HD>(p, (int)blockIdx.x - n_lg, smem);
        else pool_v<0, HD>(p, (int)blockIdx.x - n_lg, smem);
        return;
    }
    // workgroup g runs on XCD g % 8; head bh's tiles all go to XCD bh % 8
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int hm = slot / tiles_per_head;
    const int bh = xcd + 8 * hm;
    if (bh >= p.BH) return;
    const int row0 = (slot - hm * tiles_per_head) * kRT;
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float tau = (float)(1.0 / __builtin_sqrt((double)p.dscale));
    const int ntile = (nb + kCT - 1) / kCT;
    const LogitsLds L = logits_lds(nb, HD);
    float* qS = reinterpret_cast<float*>(smem + L.qS);
    float* kS = reinterpret_cast<float*>(smem + L.kS);
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    const float* qh = p.qhat + (size_t)bh * nb * HD;
    const float* kh = p.khat + (size_t)bh * nb * HD;
    const int* cnt = p.cnt + (size_t)b * nb;
    const int ra = row0 + 2 * wave, rb = ra + 1;

    // every global load of the prologue first, then the LDS stores
    constexpr int kKLoads = kCT * (HD / 4) / kLgThreads;   // float4s of one khat tile per thread
    float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 kv[kKLoads];
    float sc[kMaxColTiles][4];   // logits of (ra, j), (ra, j + 64), (rb, j), (rb, j + 64), j = 128 t + lane
    int2 cj[kMaxColTiles];       // counts of key blocks j and j + 64
    if (!kGiven) {
        if (tid < kRT * HD / 4) {
            const int r = tid / (HD / 4), c4 = (tid % (HD / 4)) * 4;
            if (row0 + r < nb) qv = *reinterpret_cast<const float4*>(qh + (size_t)(row0 + r) * HD + c4);
        }
        fetch_khat<HD>(kh, 0, nb, kv);
    }
#pragma unroll
    for (int t = 0; t < kMaxColTiles; t++) {
        const int j = t * kCT + lane;
        cj[t].x = (t < ntile && j < nb) ? cnt[j] : 0;
        cj[t].y = (t < ntile && j + 64 < nb) ? cnt[j + 64] : 0;
        if (kGiven) {
            const float* S = p.logits + (size_t)bh * nb * nb;
            sc[t][0] = (t < ntile && ra < nb && j < nb) ? S[(size_t)ra * nb + j] : 0.f;
            sc[t][1] = (t < ntile && ra < nb && j + 64 < nb) ? S[(size_t)ra * nb + j + 64] : 0.f;
            sc[t][2] = (t < ntile && rb < nb && j < nb) ? S[(size_t)rb * nb + j] : 0.f;
            sc[t][3] = (t < ntile && rb < nb && j + 64 < nb) ? S[(size_t)rb * nb + j + 64] : 0.f;
        }
    }
    const int cia = ra < nb ? cnt[ra] : 0, cib = rb < nb ? cnt[rb] : 0;
    for (int x = tid; x < kHistBins; x += kLgThreads) hist[x] = 0u;
    if (!kGiven && tid < kRT * HD / 4) {
        const int r = tid / (HD / 4), c4 = (tid % (HD / 4)) * 4;
        *reinterpret_cast<float4*>(qS + r * kHatStride + c4) = qv;
    }
    __syncthreads();

    // logits, one column tile at a time: kS[jj][c] = khat[128 t + jj][c]
    if (!kGiven) {
        const float* qa = qS + (2 * wave) * kHatStride;
        const float* qb = qa + kHatStride;
        const float* k0 = kS + lane * kHatStride;
        const float* k1 = kS + (lane + 64) * kHatStride;
#pragma unroll
        for (int t = 0; t < kMaxColTiles; t++) {
            if (t < ntile) {
                if (t > 0) __syncthreads();
#pragma unroll
                for (int e = 0; e < kKLoads; e++) {
                    const int x = tid + e * kLgThreads;
                    *reinterpret_cast<float4*>(kS + (x / (HD / 4)) * kHatStride + (x % (HD / 4)) * 4) = kv[e];
                }
                __syncthreads();
                if (t + 1 < ntile) fetch_khat<HD>(kh, (t + 1) * kCT, nb, kv);   // in flight during this tile
                float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
#pragma unroll 4
                for (int c = 0; c < HD; c += 4) {
                    const float4 x0 = *reinterpret_cast<const float4*>(k0 + c);
                    const float4 x1 = *reinterpret_cast<const float4*>(k1 + c);
                    const float4 ya = *reinterpret_cast<const float4*>(qa + c);
                    const float4 yb = *reinterpret_cast<const float4*>(qb + c);
                    a00 = __builtin_fmaf(ya.x, x0.x, a00);
                    a01 = __builtin_fmaf(ya.x, x1.x, a01);
                    a10 = __builtin_fmaf(yb.x, x0.x, a10);
                    a11 = __builtin_fmaf(yb.x, x1.x, a11);
                    a00 = __builtin_fmaf(ya.y, x0.y, a00);
                    a01 = __builtin_fmaf(ya.y, x1.y, a01);
                    a10 = __builtin_fmaf(yb.y, x0.y, a10);
                    a11 = __builtin_fmaf(yb.y, x1.y, a11);
                    a00 = __builtin_fmaf(ya.z, x0.z, a00);
                    a01 = __builtin_fmaf(ya.z, x1.z, a01);
                    a10 = __builtin_fmaf(yb.z, x0.z, a10);
                    a11 = __builtin_fmaf(yb.z, x1.z, a11);
                    a00 = __builtin_fmaf(ya.w, x0.w, a00);
                    a01 = __builtin_fmaf(ya.w, x1.w, a01);
                    a10 = __builtin_fmaf(yb.w, x0.w, a10);
                    a11 = __builtin_fmaf(yb.w, x1.w, a11);
                }
                sc[t][0] = a00 * tau;
                sc[t][1] = a01 * tau;
                sc[t][2] = a10 * tau;
                sc[t][3] = a11 * tau;
            }
        }
    }

    // row maxima over non-empty key blocks (exact: max does not round)
    float ma = -__builtin_inff(), mb = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < kMaxColTiles; t++) {
        if (cj[t].x > 0) {
            ma = fmaxf(ma, sc[t][0]);
            mb = fmaxf(mb, sc[t][2]);
        }
        if (cj[t].y > 0) {
            ma = fmaxf(ma, sc[t][1]);
            mb = fmaxf(mb, sc[t][3]);
        }
    }
    ma = wave_max(ma);
    mb = wave_max(mb);

    // scores -> keys and the histogram of their top 12 bits; logits, keys and
    // maxima out
    float* Sg = p.logits + (size_t)bh * nb * nb;
    uint32_t* Kg = p.keys + (size_t)bh * nb * nb;
    const int pf = p.prior_first, pd = p.prior_diag;
    const bool raw = p.rank_raw != 0, exact = p.band_exact != 0;
#pragma unroll
    for (int t = 0; t < kMaxColTiles; t++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int i = q < 2 ? ra : rb, j = t * kCT + lane + 64 * (q & 1);
            if (t < ntile && i < nb && j < nb) {
                const float sv = sc[t][q];
                if (!kGiven) Sg[(size_t)i * nb + j] = sv;
                const int cjq = (q & 1) ? cj[t].y : cj[t].x;
                const float s = cell_score(sv, q < 2 ? ma : mb, i, j, (q < 2 ? cia : cib) > 0, cjq > 0, pf, pd, raw,
                                           exact);
                const uint32_t key = float_key(s);
                Kg[(size_t)i * nb + j] = key;
                atomicAdd(&hist[key >> (32 - kHistBits)], 1u);
            }
        }
    }
    if (lane == 0) {
        if (ra < nb) p.rowmax[(size_t)bh * nb + ra] = ma;
        if (rb < nb) p.rowmax[(size_t)bh * nb + rb] = mb;
    }

    __syncthreads();
    uint32_t* gh = p.hist + (size_t)bh * kHistBins;
    for (int x = tid; x < kHistBins; x += kLgThreads)
        if (hist[x]) atomicAdd(&gh[x], hist[x]);
}

// ---------------------------------------------------------------- low-res sums
// Full mode, [MRA] "第四步": the low-resolution attention of 64 block rows of
// head bh over every key block, selected or not,
//   lo_all_i = sum_j w_ij vhat_j,  ll_all_i = sum_j w_ij,  w_ij = cnt_j exp(S_ij - m_i),
// from which the block attention later takes the selected cells back out.
// These workgroups ride in the selector's launch: they need only the logits
// kernel's output, so they run on the CUs the per-head selectors leave idle
// (64 rows a workgroup, so that at N = 16384 they and the selectors fit one
// round of one workgroup per CU).  Key blocks go by tiles of kKT: the
// workgroup forms the tile's weights (thread t: row t / 16, keys t % 16 +
// 16 m) and stages the tile's vhat rows, then the product runs on
// v_mfma_f32_16x16x4f32: wave w takes the 16-row tile w / 4 and the
// 16-channel tiles w % 4 + 4 x; A lane l holds W[l % 16][k = l / 16], B lane
// l holds vhat[k = l / 16][l % 16], and accumulator e of lane l is row
// 4 (l / 16) + e, channel l % 16.
constexpr int kLoRows = 64;
// key blocks per tile: 128 for 64-channel heads, 64 for 128
__host__ __device__ constexpr int lowres_keys(int hd) { return hd == 64 ? kCT : kCT / 2; }
// floats per weight-tile row (4 of pad: the 16 rows an MFMA operand reads
// start 4 banks apart)
__host__ __device__ constexpr int wt_stride(int hd) { return lowres_keys(hd) + 4; }

__host__ __device__ inline size_t lowres_lds(int /*nb*/, int hd) {
    return align16((size_t)kLoRows * wt_stride(hd) * 4) + align16((size_t)lowres_keys(hd) * hat_stride(hd) * 4);
}

template <int HD>
__device__ __forceinline__ void lowres_rows(const Params& p, int bh, int row0, unsigned char* smem) {
    constexpr int kVtStride = hat_stride(HD);
    constexpr int kKT = lowres_keys(HD);     // key blocks per tile
    constexpr int kWS = wt_stride(HD);
    constexpr int kCTW = HD / 64;            // 16-channel tiles per wave
    constexpr int kM = kKT / 16;             // weights per thread and tile
    const int nb = p.nb;
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float* wl = reinterpret_cast<float*>(smem);
    float* vt = reinterpret_cast<float*>(smem + align16((size_t)kLoRows * kWS * 4));
    const float* S = p.logits + (size_t)bh * nb * nb;
    const float* vh = p.vhat + (size_t)bh * nb * HD;
    const int* cnt = p.cnt + (size_t)b * nb;
    constexpr int kVLoads = kKT * (HD / 4) / kSelThreads;   // float4s of one vhat tile per thread
    const int r = tid >> 4, kq = tid & 15;                   // this thread's row and first key of a tile
    const int row = row0 + r;
    const bool rok = row < nb;

    // a tile's inputs: vhat rows, and this thread's logits and key counts
    float4 vv[kVLoads];
    float sv[kM];
    int cv[kM];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int e = 0; e < kVLoads; e++) {
            const int x = tid + e * kSelThreads, j = j0 + x / (HD / 4);
            vv[e] = j < nb ? *reinterpret_cast<const float4*>(vh + (size_t)j * HD + (x % (HD / 4)) * 4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int m = 0; m < kM; m++) {
            const int j = j0 + kq + 16 * m;
            cv[m] = j < nb ? cnt[j] : 0;
            sv[m] = (rok && j < nb) ? S[(size_t)row * nb + j] : 0.f;
        }
    };
    fetch(0);
    const float mrow = rok ? p.rowmax[(size_t)bh * nb + row] : 0.f;
    float lsum = 0.f;
    // wave w: row tile w / 4, 16-channel tiles w % 4 + 4 x
    const int rt = wave >> 2, ct = wave & 3;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 acc[kCTW];
#pragma unroll
    for (int x = 0; x < kCTW; x++) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < nb; j0 += kKT) {
        __syncthreads();   // every wave is done with the previous tile
#pragma unroll
        for (int m = 0; m < kM; m++) {
            const int j = j0 + kq + 16 * m;
            const float w = (rok && j < nb) ? lowres_weight(sv[m], mrow, cv[m]) : 0.f;
            wl[r * kWS + kq + 16 * m] = w;
            lsum += w;
        }
#pragma unroll
        for (int e = 0; e < kVLoads; e++) {
            const int x = tid + e * kSelThreads;
            *reinterpret_cast<float4*>(vt + (x / (HD / 4)) * kVtStride + (x % (HD / 4)) * 4) = vv[e];
        }
        __syncthreads();
        if (j0 + kKT < nb) fetch(j0 + kKT);   // in flight during this tile
        const float* wa = wl + (rt * 16 + (lane & 15)) * kWS + (lane >> 4);
        const float* vb = vt + (lane >> 4) * kVtStride + ct * 16 + (lane & 15);
#pragma unroll
        for (int k4 = 0; k4 < kKT; k4 += 4) {
            const float a = wa[k4];
#pragma unroll
            for (int x = 0; x < kCTW; x++)
                acc[x] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, vb[k4 * kVtStride + 64 * x], acc[x], 0, 0, 0);
        }
    }
    // the row's weight sum over its 16 threads (lanes 16 (l / 16) .. + 15 of the wave)
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o, 16);
    if (kq == 0 && rok) p.ll_all[(size_t)bh * nb + row] = lsum;
#pragma unroll
    for (int x = 0; x < kCTW; x++) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int orow = row0 + rt * 16 + 4 * (lane >> 4) + e;
            if (orow < nb) p.lo_all[((size_t)bh * nb + orow) * HD + (ct + 4 * x) * 16 + (lane & 15)] = acc[x][e];
        }
    }
}

// ---------------------------------------------------------------- premark
// The selector's marking pass for long heads (premarked(nb)), one workgroup
// per tile of kTileCells cells.  Every workgroup of a head makes the
// selector's first bin pick on the head's histogram (the same pick in each),
// then marks its tile: a cell whose top 12 key bits are above the bin is
// selected for sure, and a wave's 64 consecutive cells are two whole words
// of the head's selection bitmap, stored as they are; a cell inside the bin
// is appended to the head's candidate list in memory (one atomic per
// workgroup on the head's counter, which has a cache line of its own).
// When the bin holds more than kCap cells the workgroups store nothing and
// the selector walks the cells itself.
__global__ __launch_bounds__(kSelThreads) void premark_kernel(Params p) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t scan32[kSelWaves + 1];
    __shared__ uint32_t small[32];
    __shared__ uint32_t wtot[kSelWaves + 1];
    const int nb = p.nb, words = p.words;
    const uint32_t ncell = (uint32_t)nb * (uint32_t)nb;
    const int ntiles = (int)((ncell + kTileCells - 1) / kTileCells);
    // workgroup g runs on XCD g % 8: the tiles of head bh go to XCD bh % 8
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int hm = slot / ntiles, t = slot - hm * ntiles;
    const int bh = xcd + 8 * hm;
    if (bh >= p.BH) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t base = (uint32_t)t * kTileCells;
    const uint32_t* G = p.keys + (size_t)bh * ncell;

    constexpr int kPer = kHistBins / kSelThreads;
    uint32_t hv[kPer], kv[kCells];
#pragma unroll
    for (int e = 0; e < kPer; e++) hv[e] = p.hist[(size_t)bh * kHistBins + tid + e * kSelThreads];
    fetch_keys(G, base, ncell, kv);
#pragma unroll
    for (int e = 0; e < kPer; e++) hist[tid + e * kSelThreads] = hv[e];
    __syncthreads();
    const BinPick bp = pick_bin(hist, (uint32_t)p.K, scan32, small);
    if (bp.count > (uint32_t)kCap) return;

    const uint32_t p32 = bp.bin, sh = 32 - kHistBits;
    const uint32_t magic = 0xFFFFFFFFu / (uint32_t)nb + 1u;
    const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane(tid - lane);
    uint32_t* gbits = p.selbits + (size_t)bh * nb * words;
    uint64_t mh[kCells];
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < kCells; e++) {
        const uint32_t x0 = base + wbase + (uint32_t)e * kSelThreads;   // the wave's first cell (uniform)
        mh[e] = 0;
        if (x0 < ncell) {   // ncell is a multiple of 64: the group is whole
            const uint32_t top = kv[e] >> sh;
            const uint64_t ms = __ballot(top > p32);
            mh[e] = __ballot(top == p32);
            const uint32_t i0 = row_of(x0, (uint32_t)nb, magic), j0 = x0 - i0 * (uint32_t)nb;
            if (lane == 0)
                *reinterpret_cast<uint2*>(gbits + i0 * words + (j0 >> 5)) = make_uint2((uint32_t)ms, (uint32_t)(ms >> 32));
            tot += (uint32_t)__popcll(mh[e]);
        }
    }
    // the workgroup's place in the candidate list: waves in order, one atomic
    if (lane == 0) wtot[wave] = tot;
    __syncthreads();
    if (tid == 0) {
        uint32_t acc = 0;
        for (int w = 0; w < kSelWaves; w++) {
            const uint32_t c = wtot[w];
            wtot[w] = acc;
            acc += c;
        }
        wtot[kSelWaves] = acc ? atomicAdd(&p.ncand[(size_t)bh * kCandStride], acc) : 0u;
    }
    __syncthreads();
    if (tot) {
        uint32_t at0 = wtot[kSelWaves] + wtot[wave];
        const uint64_t lt_mask = (1ull << lane) - 1ull;
        uint64_t* gc = p.cand + (size_t)bh * kCap;
#pragma unroll
        for (int e = 0; e < kCells; e++) {
            if ((mh[e] >> lane) & 1ull) {
                const uint32_t at = at0 + (uint32_t)__popcll(mh[e] & lt_mask);
                if (at < (uint32_t)kCap) gc[at] = cell_key64(kv[e], base + wbase + (uint32_t)e * kSelThreads + lane);
            }
            at0 += (uint32_t)__popcll(mh[e]);
        }
    }
}

// ---------------------------------------------------------------- select
// ---------------------------------------------------------------- stream
// Head bh's selection, given as its bitmap in LDS (nb rows of `words`
// words), into what the attention and join kernels read: the CSR (row_ptr,
// col), the bitmap in memory, the segment pointers, the rows the join
// kernel combines and one record per selected block.  mbv: the blocks' mask
// words in LDS (written before the call; read after its barriers).  wp: LDS
// for nb * words 16-bit counts (each bitmap word's set bits before it in its
// row).  expect: the number of selected cells the caller made (the error
// word's bit 2 flags another count), or -1 when the count is the layout's
// own (it must stay within the stream's capacity p.K).  Called by a whole
// kSelThreads workgroup.
__device__ __forceinline__ void emit_stream(const Params& p, int bh, const uint32_t* bitmap, const uint32_t* mbv, int* rc,
                            int* ic, uint64_t* scan64, uint16_t* wp, int64_t expect) {
    const int nb = p.nb, words = p.words;
    const int tid = threadIdx.x;
    // CSR row pointers, segment (item) pointers and the rows the final kernel
    // combines, in one scan: one block row per thread (nb <= 512)
    int32_t* row_ptr = p.row_ptr + (size_t)bh * (nb + 1);
    int32_t* item_ptr = p.item_ptr + (size_t)bh * (nb + 1);
    {
        const int i = tid;
        int c = 0;
        if (i < nb)
            for (int w = 0; w < words; w++) {
                wp[i * words + w] = (uint16_t)c;
                c += __popc(bitmap[i * words + w]);
            }
        const int sl = row_seg_len(c, p.seg_whole, p.chunk);
        const int it = c > 0 ? (c + sl - 1) / sl : 0;
        const int mf = (i < nb && it != 1) ? 1 : 0;   // no selected block, or several segments
        const uint64_t v = (uint64_t)c | ((uint64_t)it << 32) | ((uint64_t)mf << 48);
        uint64_t tot;
        const uint64_t ex = block_excl_scan<uint64_t>(v, scan64, &tot);
        const int ec = (int)(uint32_t)ex, ei = (int)((ex >> 32) & 0xFFFFu), em = (int)(ex >> 48);
        if (i < nb) {
            row_ptr[i] = ec;
            item_ptr[i] = ei;
            rc[i] = ec;
            ic[i] = ei;
            p.join_cnt[(size_t)bh * nb + i] = 0u;
            if (mf) p.merge_rows[(size_t)bh * nb + em] = make_int4(i, ei, it, 0);
        }
        if (tid == 0) {
            const int tc = (int)(uint32_t)tot, ti = (int)((tot >> 32) & 0xFFFFu), tm = (int)(tot >> 48);
            row_ptr[nb] = tc;
            item_ptr[nb] = ti;
            rc[nb] = tc;
            ic[nb] = ti;
            p.n_merge[bh] = tm;
            if ((expect >= 0 ? (int64_t)tc != expect : (int64_t)tc > p.K) || ti > p.max_items) atomicOr(reinterpret_cast<unsigned int*>(p.error), 2u);
        }
    }
    __syncthreads();

    // the bitmap in memory
    uint32_t* gbits = p.selbits + (size_t)bh * nb * words;
    for (int x = tid; x < nb * words; x += kSelThreads) gbits[x] = bitmap[x];
    // column lists and the attention stream records: one thread per bitmap
    // word (x = i * words + w), or per half of one (hf) when the halves
    // still fit the workgroup, for its set bits in order; the k-th set bit
    // of word x is cell rc[i] + wp[x] + k of the stream.
    int32_t* col = p.col + (size_t)bh * p.K;
    BlkRec* recs = p.recs + (size_t)bh * p.K;
    const int tcap = (int)min((int64_t)rc[nb], p.K);
    const int halves = 2 * nb * words <= kSelThreads ? 1 : 0;
    for (int hx = tid; hx < (nb * words) << halves; hx += kSelThreads) {
        const int x = hx >> halves, hf = hx & halves;
        const uint32_t word = bitmap[x];
        uint32_t bits = halves ? (hf ? word >> 16 : word & 0xFFFFu) : word;
        if (bits == 0u) continue;
        const int i = x / words, w = x - i * words;
        const int o = rc[i], n = rc[i + 1] - o;
        const int ch = row_seg_len(n, p.seg_whole, p.chunk);
        const bool whole = n <= ch;
        const int rank0 = wp[x] + (hf ? __popc(word & 0xFFFFu) : 0);
        // the first bit's segment and position; later bits step them
        int sg = rank0 / ch, pos = rank0 - sg * ch;
        int item = ic[i] + sg, len = min(ch, n - sg * ch);
        int e = o + rank0;
        while (bits != 0u) {
            const int j = w * 32 + 16 * hf + __builtin_ctz(bits);
            bits &= bits - 1u;
            if (e < tcap) {
                col[e] = j;
                recs[e] = BlkRec{rec_ij(i, j), mbv[j], 0u, rec_info(item, pos, len, whole)};
            }
            e++;
            if (++pos == ch) {
                pos = 0;
                item++;
                sg++;
                len = min(ch, n - sg * ch);
            }
        }
    }
}

// The bin pick of pick_bin by wave 0 alone, so that the other waves wait at
// one barrier instead of a workgroup scan's three: lane l sums bins
// (63 - l) * 64 .. + 63 (read as 16-byte pieces), a wave scan finds the lane
// whose range holds the need-th cell from the top, and a second scan over
// that lane's 64 bins, one per lane, finds the bin.  The whole workgroup
// calls this.
__device__ __forceinline__ BinPick pick_bin_wave(const uint32_t* h, uint32_t need, uint32_t* small) {
    constexpr int kPer = kHistBins / 64;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const uint4* hv = reinterpret_cast<const uint4*>(h + (63 - lane) * kPer);
        uint32_t local = 0;
        // lane l starts its range at quad l % 16, so that the lanes of one
        // read fall on different LDS banks
#pragma unroll
        for (int e = 0; e < kPer / 4; e++) {
            const uint4 c = hv[(e + lane) & (kPer / 4 - 1)];
            local += c.x + c.y + c.z + c.w;
        }
        const uint32_t above = wave_scan_incl(local) - local;
        const uint64_t hit = __ballot(above < need && need <= above + local);
        if (hit) {
            const int src = __builtin_ctzll(hit);
            const uint32_t sabove = (uint32_t)__builtin_amdgcn_readlane((int)above, src);
            const int bin = (63 - src) * kPer + (kPer - 1 - lane);   // lane 0: that range's top bin
            const uint32_t c = h[bin];
            const uint32_t ab = sabove + wave_scan_incl(c) - c;
            if (ab < need && need <= ab + c) {
                small[0] = (uint32_t)bin;
                small[1] = ab;
                small[2] = c;
            }
        }
    }
    __syncthreads();
    BinPick r{small[0], small[1], small[2]};
    return r;
}

// Position of the n-th (1-based) set bit of m.
__device__ __forceinline__ int nth_set_bit(uint64_t m, uint32_t n) {
    int pos = 0;
#pragma unroll
    for (int half = 32; half > 0; half >>= 1) {
        const uint64_t low = m & ((1ull << half) - 1ull);
        const uint32_t c = (uint32_t)__popcll(low);
        if (n > c) {
            n -= c;
            m >>= half;
            pos += half;
        } else {
            m = low;
        }
    }
    return pos;
}

// The threshold key T: the need-th largest of the candidates whose top pbits
// key bits are `prefix`.  While more than kRankSet of them remain, digit
// passes narrow the prefix (every thread adds its candidates to a 256-bin
// histogram, wave 0 picks the digit); then the remaining ones, at most
// kRankSet, are gathered and ranked pairwise by the whole workgroup (all
// keys differ, since each holds its flat index), and T is the one of rank
// need - 1.  The whole workgroup calls this; every thread gets T.
__device__ __forceinline__ uint64_t threshold_key(const uint64_t* cand, uint32_t ncand, uint64_t prefix, int pbits,
                                                  uint32_t need, uint32_t count, uint32_t* dig, uint64_t* few,
                                                  uint32_t* rank, uint32_t* small) {
    const int tid = threadIdx.x, lane = tid & 63;
    auto matches = [&](uint64_t k64) { return pbits == 64 ? k64 == prefix : (k64 >> (64 - pbits)) == prefix; };
    while (count > (uint32_t)kRankSet && pbits < 64) {
        const int db = (64 - pbits) < kDigitBits ? (64 - pbits) : kDigitBits;
        if (tid < kDigitBins) dig[tid] = 0u;
        __syncthreads();
        for (uint32_t c0 = 0; c0 < ncand; c0 += kSelThreads) {
            const uint32_t c = c0 + tid;
            bool hit = false;
            uint32_t dg = 0;
            if (c < ncand) {
                const uint64_t k64 = cand[c];
                hit = matches(k64);
                dg = (uint32_t)((k64 >> (64 - pbits - db)) & ((1ull << db) - 1));
            }
            // a wave whose hits share one digit (tie-heavy scores) adds them
            // with one atomic instead of one per lane on the same bin
            const uint64_t m = __ballot(hit);
            if (m) {
                const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)dg, __builtin_ctzll(m));
                if (__ballot(hit && dg != d0) == 0) {
                    if (lane == 0) atomicAdd(&dig[d0], (uint32_t)__popcll(m));
                } else if (hit) {
                    atomicAdd(&dig[dg], 1u);
                }
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane l: bins 4 (63 - l) + 3 .. 4 (63 - l), from the top
            const uint4 c4 = reinterpret_cast<const uint4*>(dig)[63 - lane];
            const uint32_t cb[4] = {c4.w, c4.z, c4.y, c4.x};
            const uint32_t local = c4.x + c4.y + c4.z + c4.w;
            uint32_t acc = wave_scan_incl(local) - local;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                if (acc < need && need <= acc + cb[q]) {
                    small[16] = (uint32_t)(4 * (63 - lane) + 3 - q);
                    small[17] = acc;
                    small[18] = cb[q];
                }
                acc += cb[q];
            }
        }
        __syncthreads();
        need -= small[17];
        prefix = (prefix << db) | small[16];
        pbits += db;
        count = small[18];
    }
    // gather the remaining candidates (at most kRankSet) and rank them
    if (tid == 0) small[24] = 0u;
    if (tid < kRankSet) rank[tid] = 0u;
    __syncthreads();
    for (uint32_t c0 = 0; c0 < ncand; c0 += kSelThreads) {
        const uint32_t c = c0 + tid;
        const bool hit = c < ncand && matches(cand[c]);
        const uint64_t m = __ballot(hit);
        if (m) {
            uint32_t at = 0;
            if (lane == 0) at = atomicAdd(&small[24], (uint32_t)__popcll(m));
            at = (uint32_t)__builtin_amdgcn_readfirstlane((int)at) + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
            if (hit && at < (uint32_t)kRankSet) few[at] = cand[c];
        }
    }
    __syncthreads();
    const uint32_t nf = small[24] < (uint32_t)kRankSet ? small[24] : (uint32_t)kRankSet;
    {
        // thread (j, l): does few[j] outrank few[l]?  four j per thread
        const uint32_t l = (uint32_t)tid & 63u;
        uint32_t r = 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const uint32_t j = ((uint32_t)tid >> 6) + 16u * q;
            if (j < nf && l < nf && few[j] > few[l]) r++;
        }
        if (r) atomicAdd(&rank[l], r);
    }
    __syncthreads();
    if (tid < 64) {
        const bool is_t = (uint32_t)tid < nf && rank[tid] == need - 1u;
        const uint64_t m = __ballot(is_t);
        if (tid == 0) {
            const uint64_t T = m ? few[__builtin_ctzll(m)] : (pbits == 64 ? prefix : prefix << (64 - pbits));
            small[20] = (uint32_t)(T >> 32);
            small[21] = (uint32_t)T;
        }
    }
    __syncthreads();
    return ((uint64_t)small[20] << 32) | small[21];
}

// The marking pass of select_rows over every cell of a one-tile head of
// 1 << kLnb block rows (kv: the thread's cell keys, cell tid + e * kSelThreads
// in kv[e]; a wave's 64 consecutive cells, group g = e * kSelWaves + wave, lie
// in one block row).  Cells whose key prefix is above `prefix` are selected
// for sure: their count goes to gcnt[g], and the workgroup's own rows (row0 ..
// + kTileRows) get their bitmap words.  Cells whose prefix equals it are
// candidates: each wave places its own with one LDS atomic on small[8].
// kNarrow: the prefix has at most 32 bits (a prefix of the score key alone).
// Per group the loop only takes the two ballots: the sure-cell ballot goes
// into lane e of two registers, and after the loop each lane e < kCells
// counts and stores group e's, so that the scalar unit, which the 16 waves
// of the workgroup share, does one popcount per group.
template <bool kNarrow, int kLnb>
__device__ __forceinline__ void mark_groups(const uint32_t (&kv)[kCells], int words, int row0, uint64_t prefix,
                                            int pbits, uint32_t* gcnt, uint32_t* bitmap, uint64_t* cand,
                                            uint32_t* small) {
    constexpr int kNb = 1 << kLnb;
    constexpr int kE = kNb * kNb / kSelThreads < kCells ? kNb * kNb / kSelThreads : kCells;   // groups with cells
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)threadIdx.x - lane);
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    // narrow prefix: top = key >> sh is above p32 when key > hi, and equal
    // to it when key >= lo and not above
    const uint32_t sh = kNarrow ? (uint32_t)(32 - pbits) : 0u, p32 = (uint32_t)prefix;
    const uint32_t lo = kNarrow ? p32 << sh : 0u;
    const uint32_t hi = kNarrow ? (uint32_t)((((uint64_t)p32 + 1u) << sh) - 1u) : 0u;
    uint64_t mh[kE];
    uint32_t s_lo = 0u, s_hi = 0u, tot = 0;
    static_for<0, kE>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        uint64_t ms;
        if constexpr (kNarrow) {
            ms = __ballot(kv[e] > hi);
            mh[e] = __ballot(kv[e] >= lo) & ~ms;
        } else {
            const uint64_t top = cell_key64(kv[e], (uint32_t)e * kSelThreads + wbase + lane) >> (64 - pbits);
            ms = __ballot(top > prefix);
            mh[e] = __ballot(top == prefix);
        }
        s_lo = write_lane<e>(s_lo, (uint32_t)ms);
        s_hi = write_lane<e>(s_hi, (uint32_t)(ms >> 32));
        tot += (uint32_t)__popcll(mh[e]);
    });
    if (lane < kCells) {
        gcnt[lane * kSelWaves + wave] = (uint32_t)(__popc(s_lo) + __popc(s_hi));   // 0 past the head's cells
        const uint32_t x0 = (uint32_t)lane * kSelThreads + wbase;
        const uint32_t r = (x0 >> kLnb) - (uint32_t)row0;
        if (r < (uint32_t)kTileRows)
            *reinterpret_cast<uint2*>(bitmap + r * words + ((x0 & (uint32_t)(kNb - 1)) >> 5)) = make_uint2(s_lo, s_hi);
    }
    if (tot) {
        uint32_t at = 0;
        if (lane == 0) at = atomicAdd(&small[8], tot);
        at = (uint32_t)__builtin_amdgcn_readfirstlane((int)at);
#pragma unroll
        for (int e = 0; e < kE; e++) {
            if (mh[e]) {
                if ((mh[e] >> lane) & 1ull) {
                    const uint32_t pos = at + (uint32_t)__popcll(mh[e] & lt_mask);
                    if (pos < (uint32_t)kCap) cand[pos] = cell_key64(kv[e], (uint32_t)e * kSelThreads + wbase + lane);
                }
                at += (uint32_t)__popcll(mh[e]);
            }
        }
    }
}

// ---------------------------------------------------------------- select by row tiles
// One-tile heads whose block rows hold whole 64-cell groups (nb = 64 or 128,
// N = 2048 or 4096) are selected by nb / kTileRows workgroups per head, all
// on the head's XCD.  Every workgroup of a head makes the same decisions for
// the whole head from the same inputs (the head's histogram and every cell
// key, read from the head's L2): the threshold bin, the candidates, the
// threshold key T and the selected count of every 64-cell group.  It then
// writes only its own rows' share of the output: their bitmap words, row and
// segment pointers, join-list entries and records.  No workgroup waits for
// another.
__device__ __forceinline__ void select_rows(const Params& p, int bh, int t, unsigned char* smem) {
    const int nb = p.nb, words = p.words;
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row0 = t * kTileRows;
    const int lnb = nb == 128 ? 7 : 6;   // log2(nb)
    const TileLds L = tile_lds(nb);
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    uint32_t* dig = reinterpret_cast<uint32_t*>(smem + L.dig);
    uint64_t* cand = reinterpret_cast<uint64_t*>(smem + L.cand);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + L.bitmap);
    int* rc = reinterpret_cast<int*>(smem + L.rc);
    int* ic = reinterpret_cast<int*>(smem + L.ic);
    uint32_t* mbv = reinterpret_cast<uint32_t*>(smem + L.mbv);
    uint32_t* gcnt = reinterpret_cast<uint32_t*>(smem + L.wcnt);   // per 64-cell group g = e * kSelWaves + wave
    uint64_t* few = reinterpret_cast<uint64_t*>(smem + L.few);
    uint32_t* rank = reinterpret_cast<uint32_t*>(smem + L.rank);
    uint32_t* small = reinterpret_cast<uint32_t*>(smem + L.small);
    const uint32_t ncell = (uint32_t)nb * (uint32_t)nb;
    const uint32_t* G = p.keys + (size_t)bh * ncell;

    // prologue: every global load first
    constexpr int kPer = kHistBins / kSelThreads;
    uint32_t hv[kPer], kv[kCells];
#pragma unroll
    for (int e = 0; e < kPer; e++) hv[e] = p.hist[(size_t)bh * kHistBins + tid + e * kSelThreads];
    fetch_keys(G, 0, ncell, kv);
    const uint32_t mv = tid < nb ? p.mbits[b * nb + tid] : 0u;
#pragma unroll
    for (int e = 0; e < kPer; e++) hist[tid + e * kSelThreads] = hv[e];
    if (tid < kTileRows * words) bitmap[tid] = 0u;
    if (tid < nb) mbv[tid] = mv;
    if (tid == 0) small[8] = 0u;
    __syncthreads();

    uint32_t need = (uint32_t)p.K;
    BinPick bp = pick_bin_wave(hist, need, small);
    need -= bp.above;
    uint64_t prefix = bp.bin;
    int pbits = kHistBits;
    uint32_t count = bp.count;
    // further 12-bit passes while the bin is too large for LDS (tie-heavy inputs)
    while (count > (uint32_t)kCap && pbits < 64) {
        __syncthreads();   // every thread has read small[0..2]
        const int db = (64 - pbits) < 12 ? (64 - pbits) : 12;
        for (int x = tid; x < kHistBins; x += kSelThreads) hist[x] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kCells; e++) {
            const uint32_t x = tid + e * kSelThreads;
            const uint64_t k64 = cell_key64(kv[e], x);
            if (x < ncell && (k64 >> (64 - pbits)) == prefix)
                atomicAdd(&hist[(uint32_t)((k64 >> (64 - pbits - db)) & ((1ull << db) - 1))], 1u);
        }
        __syncthreads();
        bp = pick_bin_wave(hist, need, small);
        need -= bp.above;
        prefix = (prefix << db) | bp.bin;
        pbits += db;
        count = bp.count;
    }

    // One pass over every cell of the head, 64-cell groups: cells above the
    // bin are selected for sure (their count per group, and this workgroup's
    // rows' bitmap words); cells inside it are candidates, placed in the list
    // with one LDS atomic per wave.
    if (lnb == 7) {
        if (pbits <= 32) mark_groups<true, 7>(kv, words, row0, prefix, pbits, gcnt, bitmap, cand, small);
        else mark_groups<false, 7>(kv, words, row0, prefix, pbits, gcnt, bitmap, cand, small);
    } else {
        if (pbits <= 32) mark_groups<true, 6>(kv, words, row0, prefix, pbits, gcnt, bitmap, cand, small);
        else mark_groups<false, 6>(kv, words, row0, prefix, pbits, gcnt, bitmap, cand, small);
    }
    __syncthreads();
    const uint32_t ncand_all = small[8];
    const uint32_t ncand = ncand_all < (uint32_t)kCap ? ncand_all : (uint32_t)kCap;
    if (tid == 0 && ncand_all != count) atomicOr(reinterpret_cast<unsigned int*>(p.error), 1u);

    const uint64_t T = threshold_key(cand, ncand, prefix, pbits, need, count, dig, few, rank, small);
    if (tid == 0 && t == 0) p.thresh[bh] = T;

    // candidates at or above the threshold: their groups' counts, and this
    // workgroup's rows' bitmap
    for (uint32_t c = tid; c < ncand; c += kSelThreads) {
        const uint64_t k64 = cand[c];
        if (k64 >= T) {
            const uint32_t f = 0xFFFFFFFFu - (uint32_t)k64;
            if (f < ncell) {
                atomicAdd(&gcnt[f >> 6], 1u);
                const uint32_t i = f >> lnb, j = f & (uint32_t)(nb - 1);
                if (i - (uint32_t)row0 < (uint32_t)kTileRows)
                    atomicOr(&bitmap[(i - row0) * words + (j >> 5)], 1u << (j & 31));
            }
        }
    }
    __syncthreads();

    // every row's CSR and segment pointers and join flag from one scan by
    // wave 0, rows 2 lane and 2 lane + 1 (a row is nb / 64 consecutive
    // groups; the same in every workgroup of the head); this workgroup
    // writes its rows'
    int32_t* row_ptr = p.row_ptr + (size_t)bh * (nb + 1);
    int32_t* item_ptr = p.item_ptr + (size_t)bh * (nb + 1);
    if (tid < 64) {
        const int gpr = nb >> 6;   // groups per row
        int cc[2], itc[2], mfc[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int i = 2 * tid + q;
            int c = 0;
            if (i < nb) {
                c = (int)gcnt[i * gpr];
                if (gpr == 2) c += (int)gcnt[i * gpr + 1];
            }
            cc[q] = c;
            const int sl = row_seg_len(c, p.seg_whole, p.chunk);
            itc[q] = c > 0 ? (c + sl - 1) / sl : 0;
            mfc[q] = (i < nb && itc[q] != 1) ? 1 : 0;   // no selected block, or several segments
        }
        // counts in bits 0..19 and join flags in 20..31 of one word; segments in another
        const uint32_t va = (uint32_t)(cc[0] + cc[1]) | ((uint32_t)(mfc[0] + mfc[1]) << 20);
        const uint32_t vi = (uint32_t)(itc[0] + itc[1]);
        const uint32_t xa = wave_scan_incl(va), xi = wave_scan_incl(vi);
        int ec = (int)((xa - va) & 0xFFFFFu), em = (int)((xa - va) >> 20), ei = (int)(xi - vi);
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int i = 2 * tid + q;
            if (i < nb) {
                rc[i] = ec;
                ic[i] = ei;
                if ((uint32_t)(i - row0) < (uint32_t)kTileRows) {
                    row_ptr[i] = ec;
                    item_ptr[i] = ei;
                    p.join_cnt[(size_t)bh * nb + i] = 0u;
                    if (mfc[q]) p.merge_rows[(size_t)bh * nb + em] = make_int4(i, ei, itc[q], 0);
                }
            }
            ec += cc[q];
            ei += itc[q];
            em += mfc[q];
        }
        if (tid == 63) {
            const int tc = (int)(xa & 0xFFFFFu), tm = (int)(xa >> 20), ti = (int)xi;
            rc[nb] = tc;
            ic[nb] = ti;
            if (row0 + kTileRows == nb) {
                row_ptr[nb] = tc;
                item_ptr[nb] = ti;
                p.n_merge[bh] = tm;
            }
            if ((int64_t)tc != p.K || ti > p.max_items) atomicOr(reinterpret_cast<unsigned int*>(p.error), 2u);
        }
    }
    __syncthreads();

    // this workgroup's rows of the bitmap in memory; its cells' columns and
    // records, one thread per selected cell (row by binary search over the
    // row pointers, key block as the bit of the cell's rank in its row)
    uint32_t* gbits = p.selbits + ((size_t)bh * nb + row0) * words;
    if (tid < kTileRows * words) gbits[tid] = bitmap[tid];
    int32_t* col = p.col + (size_t)bh * p.K;
    BlkRec* recs = p.recs + (size_t)bh * p.K;
    const int e_end = (int)min((int64_t)rc[row0 + kTileRows], p.K);
    for (int e = rc[row0] + tid; e < e_end; e += kSelThreads) {
        int lo = row0, hi = row0 + kTileRows - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (rc[mid] <= e) lo = mid;
            else hi = mid - 1;
        }
        const int i = lo, o = rc[i], n = rc[i + 1] - o, rank_in_row = e - o;
        const uint32_t* row = bitmap + (i - row0) * words;
        int r = rank_in_row, w = 0;
        uint32_t bits = row[0];
        int c = __popc(bits);
        while (r >= c && w + 1 < words) {
            r -= c;
            bits = row[++w];
            c = __popc(bits);
        }
        const int j = w * 32 + nth_set_bit(bits, (uint32_t)r + 1u);
        col[e] = j;
        const int ch = row_seg_len(n, p.seg_whole, p.chunk), nit = (n + ch - 1) / ch, sg = rank_in_row / ch;
        const int len = min(ch, n - sg * ch);
        recs[e] = BlkRec{rec_ij(i, j), mbv[j], 0u, rec_info(ic[i] + sg, rank_in_row - sg * ch, len, nit == 1)};
    }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb;
    // (heads of 64 or 128 block rows are selected by lgsel_kernel)
    // workgroups [0, BH_pad) select, one per head (BH_pad = BH rounded up to
    // a multiple of 8, so workgroup bh runs on XCD bh % 8); in full mode the
    // rest sum the low-res attention of kLoRows rows each, placed on the XCD of
    // their head
    const int bh_pad = 8 * ((p.BH + 7) / 8);
    if ((int)blockIdx.x >= bh_pad) {
        const int g = blockIdx.x - bh_pad, xcd = g & 7, slot = g >> 3;
        const int tiles = (nb + kLoRows - 1) / kLoRows;
        const int hm = slot / tiles, lbh = xcd + 8 * hm;
        if (lbh < p.BH) {
            if (p.d == 128) lowres_rows<128>(p, lbh, (slot - hm * tiles) * kLoRows, smem);
            else lowres_rows<64>(p, lbh, (slot - hm * tiles) * kLoRows, smem);
        }
        return;
    }
    const int bh = blockIdx.x;
    if (bh >= p.BH) return;
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const SelectLds L = select_lds(nb);
    const int words = p.words;
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    uint32_t* dig = reinterpret_cast<uint32_t*>(smem + L.dig);
    uint64_t* cand = reinterpret_cast<uint64_t*>(smem + L.cand);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + L.bitmap);
    int* rc = reinterpret_cast<int*>(smem + L.rc);
    int* ic = reinterpret_cast<int*>(smem + L.ic);
    uint32_t* mbv = reinterpret_cast<uint32_t*>(smem + L.mbv);
    uint32_t* scan32 = reinterpret_cast<uint32_t*>(smem + L.scan);
    uint64_t* scan64 = reinterpret_cast<uint64_t*>(smem + L.scan);
    uint32_t* small = reinterpret_cast<uint32_t*>(smem + L.small);
    const uint32_t ncell = (uint32_t)nb * (uint32_t)nb;
    const int ntiles = (int)((ncell + kTileCells - 1) / kTileCells);
    const uint32_t* G = p.keys + (size_t)bh * ncell;
    const uint32_t magic = 0xFFFFFFFFu / (uint32_t)nb + 1u;

    // prologue: every global load first; the histogram goes to LDS at once,
    // the keys stay in registers, and the mask words (needed only for the
    // records) go to LDS later, so that their latency hides behind the
    // threshold search.  With the pre-marking pass the keys are not needed.
    const bool pre_ok = premarked(nb);
    uint32_t kv[kCells];
    constexpr int kPer = kHistBins / kSelThreads;
    uint32_t hv[kPer];
#pragma unroll
    for (int e = 0; e < kPer; e++) hv[e] = p.hist[(size_t)bh * kHistBins + tid + e * kSelThreads];
    if (!pre_ok) fetch_keys(G, 0, ncell, kv);
    const uint32_t npre = pre_ok ? p.ncand[(size_t)bh * kCandStride] : 0u;
    const uint32_t mv = tid < nb ? p.mbits[b * nb + tid] : 0u;   // nb <= 512 < kSelThreads
#pragma unroll
    for (int e = 0; e < kPer; e++) hist[tid + e * kSelThreads] = hv[e];
    for (int x = tid; x < nb * words; x += kSelThreads) bitmap[x] = 0u;
    if (tid < 2 * kDigitBins) dig[tid] = 0u;
    if (tid == 0) small[8] = 0u;
    __syncthreads();

    uint32_t need = (uint32_t)p.K;
    BinPick bp = pick_bin(hist, need, scan32, small);
    need -= bp.above;
    uint64_t prefix = bp.bin;
    int pbits = kHistBits;
    uint32_t count = bp.count;
    // the pre-marking kernel made the same bin pick and, when the bin fits
    // the candidate list, did the marking pass
    const bool pre = pre_ok && count <= (uint32_t)kCap;

    // further 12-bit passes while the bin is too large for LDS (tie-heavy inputs)
    bool tile0 = !pre_ok;   // kv holds tile 0
    while (count > (uint32_t)kCap && pbits < 64) {
        const int db = (64 - pbits) < 12 ? (64 - pbits) : 12;
        for (int x = tid; x < kHistBins; x += kSelThreads) hist[x] = 0u;
        __syncthreads();
        for (int t = 0; t < ntiles; t++) {
            const uint32_t base = (uint32_t)t * kTileCells;
            if (ntiles > 1) {
                fetch_keys(G, base, ncell, kv);
                tile0 = t == 0;
            }
#pragma unroll
            for (int e = 0; e < kCells; e++) {
                const uint32_t x = base + tid + e * kSelThreads;
                const uint64_t k64 = cell_key64(kv[e], x);
                if (x < ncell && (k64 >> (64 - pbits)) == prefix)
                    atomicAdd(&hist[(uint32_t)((k64 >> (64 - pbits - db)) & ((1ull << db) - 1))], 1u);
            }
        }
        __syncthreads();
        bp = pick_bin(hist, need, scan32, small);
        need -= bp.above;
        prefix = (prefix << db) | bp.bin;
        pbits += db;
        count = bp.count;
    }

    // One pass over the cells: cells above the bin are selected for sure
    // (bitmap), cells inside it are appended to the LDS candidate list.
    // After the pre-marking pass both come from memory instead.
    const bool rows64 = (nb & 63) == 0;
    if (pre) {
        const uint32_t* gb = p.selbits + (size_t)bh * nb * words;
        for (int x = tid; x < nb * words; x += kSelThreads) bitmap[x] = gb[x];
        const uint32_t nc = npre < (uint32_t)kCap ? npre : (uint32_t)kCap;
        const uint64_t* gc = p.cand + (size_t)bh * kCap;
        for (uint32_t c = tid; c < nc; c += kSelThreads) cand[c] = gc[c];
        if (tid == 0) small[8] = npre;
    } else {
        if (!tile0) fetch_keys(G, 0, ncell, kv);
        if (pbits <= 32 && rows64 && ncell == (uint32_t)kTileCells) {
            mark_cells_fast(nb, words, magic, (uint32_t)prefix, pbits, kv, bitmap, cand, small);
        } else if (pbits <= 32) {
            if (rows64) mark_cells<true, true>(G, ncell, ntiles, nb, words, magic, prefix, pbits, kv, bitmap, cand, small);
            else mark_cells<false, true>(G, ncell, ntiles, nb, words, magic, prefix, pbits, kv, bitmap, cand, small);
        } else {
            if (rows64) mark_cells<true, false>(G, ncell, ntiles, nb, words, magic, prefix, pbits, kv, bitmap, cand, small);
            else mark_cells<false, false>(G, ncell, ntiles, nb, words, magic, prefix, pbits, kv, bitmap, cand, small);
        }
    }
    __syncthreads();
    const uint32_t ncand_all = small[8];
    const uint32_t ncand = ncand_all < (uint32_t)kCap ? ncand_all : (uint32_t)kCap;
    if (tid == 0 && ncand_all != count) atomicOr(reinterpret_cast<unsigned int*>(p.error), 1u);

    // 8-bit passes over the candidates until the K-th largest key is pinned
    // down; the two digit histograms alternate, so a pass clears the other one
    // and needs two barriers.
    int buf = 0;
    while (pbits < 64) {
        const int db = (64 - pbits) < kDigitBits ? (64 - pbits) : kDigitBits;
        uint32_t* hc = dig + buf * kDigitBins;
        for (uint32_t c = tid; c < ncand; c += kSelThreads) {
            const uint64_t k64 = cand[c];
            if ((k64 >> (64 - pbits)) == prefix)
                atomicAdd(&hc[(uint32_t)((k64 >> (64 - pbits - db)) & ((1ull << db) - 1))], 1u);
        }
        if (tid < kDigitBins) dig[(buf ^ 1) * kDigitBins + tid] = 0u;
        __syncthreads();
        if (tid < 64) pick_digit_wave(hc, need, small + 16);
        __syncthreads();
        const uint32_t dbin = small[16], dabove = small[17], dcount = small[18];
        need -= dabove;
        prefix = (prefix << db) | dbin;
        pbits += db;
        buf ^= 1;
        if (dcount == 1u && pbits < 64) {
            // a single cell left: it is the threshold
            for (uint32_t c = tid; c < ncand; c += kSelThreads) {
                const uint64_t k64 = cand[c];
                if ((k64 >> (64 - pbits)) == prefix) {
                    small[20] = (uint32_t)(k64 >> 32);
                    small[21] = (uint32_t)k64;
                }
            }
            __syncthreads();
            prefix = ((uint64_t)small[20] << 32) | small[21];
            pbits = 64;
        }
    }
    const uint64_t T = prefix;
    if (tid == 0) p.thresh[bh] = T;

    // candidates at or above the threshold join the bitmap
    for (uint32_t c = tid; c < ncand; c += kSelThreads) {
        const uint64_t k64 = cand[c];
        if (k64 >= T) {
            const uint32_t f = 0xFFFFFFFFu - (uint32_t)k64;
            const uint32_t i = row_of(f, (uint32_t)nb, magic), j = f - i * (uint32_t)nb;
            if (i < (uint32_t)nb) atomicOr(&bitmap[i * words + (j >> 5)], 1u << (j & 31));
        }
    }
    __syncthreads();

    // the records' input, loaded in the prologue (read after the scan's barriers)
    if (tid < nb) mbv[tid] = mv;
    emit_stream(p, bh, bitmap, mbv, rc, ic, scan64, reinterpret_cast<uint16_t*>(hist), p.K);
}

// ---------------------------------------------------------------- logits and selection in one launch
// One-tile heads (row_tiled(nb): N = 2048 or 4096) run step 1's logits and
// step 2's selection in one launch, which saves a launch and its ramp between
// them.  Head bh has nb / kFusedRows workgroups, all on the head's XCD.
// Workgroup t first forms block rows 16 t .. 16 t + 15 as logits_kernel
// does (wave w: row 16 t + w; lane l: key blocks l and l + 64): logits, row
// maxima, keys and the histogram, added into the head's.  Once its stores and
// adds have completed it adds one to the head's arrival count (ncand word 1).
// Workgroups t < nb / kTileRows then wait for the count to reach every
// workgroup of the head and select rows 32 t .. 32 t + 31 (select_rows); in
// full mode the next ones then sum the low-resolution attention of 64 rows
// each (lowres_rows); the others end after their logits.
// What a workgroup stored is in its XCD's L2 once the stores have completed,
// and the waiting workgroups, on the same XCD, have not read those lines
// before, so plain loads see it.  The launch is used only when all of its
// logits workgroups are resident at once (fused_select), so every workgroup
// a head's workgroups wait for is running, and the V workgroups after them
// get the CUs that logits-only and selecting workgroups free.  The wait is
// bounded all the same: after kWaitPolls polls the workgroup sets error bit
// 32 (MRA_DEVERR_WAIT) and goes on.
constexpr int kFusedRows = kSelWaves;          // block rows per workgroup in the logits phase
constexpr uint32_t kWaitPolls = 1u << 18;
constexpr uint32_t kErrWait = 32u;

// The workgroup's stores and atomics have all completed (each thread waits
// for its own, then the barrier), then one count goes up.
__device__ __forceinline__ void arrive(uint32_t* count) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__host__ __device__ inline size_t fused_logits_lds(int hd) {
    return align16((size_t)kFusedRows * hat_stride(hd) * 4) + align16((size_t)kCT * hat_stride(hd) * 4) +
           kHistBins * 4;
}

// V pooling without staging (full mode, in lgsel_kernel): lane l of wave w
// pools channels 2 (l % (HD / 2)) and + 1 of one block, reading its 32 token
// words straight into registers (a wave's loads of one token are whole
// 128-byte rows), then sums the valid ones in token order from +0 and divides
// by the count, as pool_unit does; the block's mask word is the one pooling
// stored.  Workgroup g pools 16 * 128 / HD consecutive blocks of one head;
// returns the head, or -1 for a workgroup past the last head.
__host__ __device__ constexpr int v_direct_blocks(int hd) { return kSelWaves * (128 / hd); }
__host__ __device__ inline int v_direct_groups(int nb, int hd) {
    return (nb + v_direct_blocks(hd) - 1) / v_direct_blocks(hd);
}

template <int DT, int HD>
__device__ __forceinline__ int pool_v_direct(const Params& p, int g) {
    constexpr int kPairs = HD / 2;   // lanes per block
    const int per_head = v_direct_groups(p.nb, HD);
    const int xcd = g & 7, slot = g >> 3;
    const int hm = slot / per_head;
    const int bh = xcd + 8 * hm;
    if (bh >= p.BH) return -1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int blk = (slot - hm * per_head) * v_direct_blocks(HD) + wave * (64 / kPairs) + lane / kPairs;
    const int cp = lane % kPairs;
    if (blk < p.nb) {
        const uint32_t bits = p.mbits[(size_t)(bh / p.H) * p.nb + blk];
        float a0 = 0.0f, a1 = 0.0f;
        if constexpr (DT == 1) {
            const uint32_t* src =
                static_cast<const uint32_t*>(p.v) + ((size_t)bh * p.N + (size_t)blk * kBlock) * kPairs + cp;
            uint32_t w[kBlock];
#pragma unroll
            for (int x = 0; x < kBlock; x++) w[x] = src[(size_t)x * kPairs];
#pragma unroll
            for (int x = 0; x < kBlock; x++) {
                if ((bits >> x) & 1u) {
                    a0 = a0 + __uint_as_float(w[x] << 16);
                    a1 = a1 + __uint_as_float(w[x] & 0xFFFF0000u);
                }
            }
        } else {
            const float2* src =
                static_cast<const float2*>(p.v) + ((size_t)bh * p.N + (size_t)blk * kBlock) * kPairs + cp;
            float2 w[kBlock];
#pragma unroll
            for (int x = 0; x < kBlock; x++) w[x] = src[(size_t)x * kPairs];
#pragma unroll
            for (int x = 0; x < kBlock; x++) {
                if ((bits >> x) & 1u) {
                    a0 = a0 + w[x].x;
                    a1 = a1 + w[x].y;
                }
            }
        }
        const int count = __popc(bits);
        const float fc = (float)count;
        *reinterpret_cast<float2*>(p.vhat + ((size_t)bh * p.nb + blk) * HD + 2 * cp) =
            count > 0 ? make_float2(a0 / fc, a1 / fc) : make_float2(0.0f, 0.0f);
    }
    return bh;
}

template <bool kGiven, int HD>
__device__ __forceinline__ void fused_logits(const Params& p, int bh, int row0, unsigned char* smem) {
    constexpr int kHatStride = hat_stride(HD);
    constexpr int kKL = kCT * (HD / 4) / kSelThreads;   // float4s of the head's khat per thread (nb <= kCT)
    const int nb = p.nb;
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float tau = (float)(1.0 / __builtin_sqrt((double)p.dscale));
    float* qS = reinterpret_cast<float*>(smem);
    float* kS = reinterpret_cast<float*>(smem + align16((size_t)kFusedRows * kHatStride * 4));
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + align16((size_t)kFusedRows * kHatStride * 4) +
                                                 align16((size_t)kCT * kHatStride * 4));
    const float* qh = p.qhat + (size_t)bh * nb * HD;
    const float* kh = p.khat + (size_t)bh * nb * HD;
    const int* cnt = p.cnt + (size_t)b * nb;
    float* Sg = p.logits + (size_t)bh * nb * nb;
    // waves 0 .. 7 form the logits (the staged khat is read once per two
    // rows, which keeps the LDS reads at the pace of the fmas); wave w owns
    // rows ra = row0 + 2 w and ra + 1, lane l key blocks l and l + 64
    const bool lw = wave < kFusedRows / 2;
    const int ra = row0 + 2 * (wave & (kFusedRows / 2 - 1)), rb = ra + 1;   // < nb: nb is a multiple of 16
    const int j0 = lane, j1 = lane + 64;                                      // j0 < nb always (nb >= 64)

    // every global load of the prologue first, then the LDS stores
    float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 kv[kKL];
    float sc[4] = {0.f, 0.f, 0.f, 0.f};   // logits of (ra, j0), (ra, j1), (rb, j0), (rb, j1)
    if (!kGiven) {
        if (tid < kFusedRows * HD / 4) {
            const int r = tid / (HD / 4), c4 = (tid % (HD / 4)) * 4;
            qv = *reinterpret_cast<const float4*>(qh + (size_t)(row0 + r) * HD + c4);
        }
#pragma unroll
        for (int e = 0; e < kKL; e++) {
            const int x = tid + e * kSelThreads, jj = x / (HD / 4), c4 = (x % (HD / 4)) * 4;
            kv[e] = jj < nb ? *reinterpret_cast<const float4*>(kh + (size_t)jj * HD + c4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else if (lw) {
        sc[0] = Sg[(size_t)ra * nb + j0];
        sc[1] = j1 < nb ? Sg[(size_t)ra * nb + j1] : 0.f;
        sc[2] = Sg[(size_t)rb * nb + j0];
        sc[3] = j1 < nb ? Sg[(size_t)rb * nb + j1] : 0.f;
    }
    const int c0 = cnt[j0];
    const int c1 = j1 < nb ? cnt[j1] : 0;
    const int cia = cnt[ra], cib = cnt[rb];
    for (int x = tid; x < kHistBins; x += kSelThreads) hist[x] = 0u;
    if (!kGiven) {
        if (tid < kFusedRows * HD / 4) {
            const int r = tid / (HD / 4), c4 = (tid % (HD / 4)) * 4;
            *reinterpret_cast<float4*>(qS + r * kHatStride + c4) = qv;
        }
#pragma unroll
        for (int e = 0; e < kKL; e++) {
            const int x = tid + e * kSelThreads;
            *reinterpret_cast<float4*>(kS + (x / (HD / 4)) * kHatStride + (x % (HD / 4)) * 4) = kv[e];
        }
    }
    __syncthreads();

    if (lw) {
        // the lane's four logits, each an fma chain over the channels in order
        if (!kGiven) {
            const float* qa = qS + (ra - row0) * kHatStride;
            const float* qb = qa + kHatStride;
            const float* k0 = kS + j0 * kHatStride;
            const float* k1 = kS + j1 * kHatStride;
            float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
#pragma unroll 4
            for (int c = 0; c < HD; c += 4) {
                const float4 x0 = *reinterpret_cast<const float4*>(k0 + c);
                const float4 x1 = *reinterpret_cast<const float4*>(k1 + c);
                const float4 ya = *reinterpret_cast<const float4*>(qa + c);
                const float4 yb = *reinterpret_cast<const float4*>(qb + c);
                a00 = __builtin_fmaf(ya.x, x0.x, a00);
                a01 = __builtin_fmaf(ya.x, x1.x, a01);
                a10 = __builtin_fmaf(yb.x, x0.x, a10);
                a11 = __builtin_fmaf(yb.x, x1.x, a11);
                a00 = __builtin_fmaf(ya.y, x0.y, a00);
                a01 = __builtin_fmaf(ya.y, x1.y, a01);
                a10 = __builtin_fmaf(yb.y, x0.y, a10);
                a11 = __builtin_fmaf(yb.y, x1.y, a11);
                a00 = __builtin_fmaf(ya.z, x0.z, a00);
                a01 = __builtin_fmaf(ya.z, x1.z, a01);
                a10 = __builtin_fmaf(yb.z, x0.z, a10);
                a11 = __builtin_fmaf(yb.z, x1.z, a11);
                a00 = __builtin_fmaf(ya.w, x0.w, a00);
                a01 = __builtin_fmaf(ya.w, x1.w, a01);
                a10 = __builtin_fmaf(yb.w, x0.w, a10);
                a11 = __builtin_fmaf(yb.w, x1.w, a11);
            }
            sc[0] = a00 * tau;
            sc[1] = a01 * tau;
            sc[2] = a10 * tau;
            sc[3] = a11 * tau;
        }

        // the row maxima over non-empty key blocks (exact), then scores, keys
        // and the histogram of their top 12 bits
        float ma = -__builtin_inff(), mb = -__builtin_inff();
        if (c0 > 0) {
            ma = fmaxf(ma, sc[0]);
            mb = fmaxf(mb, sc[2]);
        }
        if (c1 > 0) {
            ma = fmaxf(ma, sc[1]);
            mb = fmaxf(mb, sc[3]);
        }
        ma = wave_max(ma);
        mb = wave_max(mb);
        uint32_t* Kg = p.keys + (size_t)bh * nb * nb;
        const int pf = p.prior_first, pd = p.prior_diag;
        const bool raw = p.rank_raw != 0, exact = p.band_exact != 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int i = q < 2 ? ra : rb, j = (q & 1) ? j1 : j0;
            if (j < nb) {
                const float sv = sc[q];
                if (!kGiven) Sg[(size_t)i * nb + j] = sv;
                const float s = cell_score(sv, q < 2 ? ma : mb, i, j, (q < 2 ? cia : cib) > 0,
                                           ((q & 1) ? c1 : c0) > 0, pf, pd, raw, exact);
                const uint32_t key = float_key(s);
                Kg[(size_t)i * nb + j] = key;
                atomicAdd(&hist[key >> (32 - kHistBits)], 1u);
            }
        }
        if (lane == 0) {
            p.rowmax[(size_t)bh * nb + ra] = ma;
            p.rowmax[(size_t)bh * nb + rb] = mb;
        }
    }
    __syncthreads();
    uint32_t* gh = p.hist + (size_t)bh * kHistBins;
    for (int x = tid; x < kHistBins; x += kSelThreads)
        if (hist[x]) atomicAdd(&gh[x], hist[x]);

    // arrive: every store and histogram add of the workgroup has completed
    // before the count goes up
    arrive(p.ncand + (size_t)bh * kCandStride + 1);
}

// Wait until `count` reaches n (bounded: p.wait_polls polls, kWaitPolls when 0).
__device__ __forceinline__ void wait_count(const Params& p, uint32_t* count, uint32_t n) {
    if (threadIdx.x == 0) {
        const uint32_t limit = p.wait_polls ? p.wait_polls : kWaitPolls;
        n += p.wait_extra;
        uint32_t polls = 0;
        while (__hip_atomic_fetch_add(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
            if (++polls >= limit) {
                atomicOr(reinterpret_cast<unsigned int*>(p.error), kErrWait);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

template <bool kGiven, int HD>
__global__ __launch_bounds__(kSelThreads) void lgsel_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb;
    const int lt = nb / kFusedRows;   // logits workgroups per head
    const int heads_per_xcd = (p.BH + 7) / 8;
    const int n_lg = 8 * heads_per_xcd * lt;
    // workgroup g runs on XCD g % 8; head bh's workgroups go to XCD bh % 8,
    // in consecutive slots
    if ((int)blockIdx.x >= n_lg) {
        // full mode: V pooled by the workgroups after the logits ones, on the
        // CUs those leave free; the low-res workgroups of the head wait for them
        const int bh = p.dtype == 1 ? pool_v_direct<1, HD>(p, (int)blockIdx.x - n_lg)
                                    : pool_v_direct<0, HD>(p, (int)blockIdx.x - n_lg);
        if (bh >= 0) arrive(p.ncand + (size_t)bh * kCandStride + 2);
        return;
    }
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int hm = slot / lt, t = slot - hm * lt;
    const int bh = xcd + 8 * hm;
    if (bh >= p.BH) return;
    fused_logits<kGiven, HD>(p, bh, t * kFusedRows, smem);
    const int nsel = nb / kTileRows;
    const int nlow = p.mode == 0 ? (nb + kLoRows - 1) / kLoRows : 0;
    if (t >= nsel + nlow) return;
    wait_count(p, p.ncand + (size_t)bh * kCandStride + 1, (uint32_t)lt);
    if (t < nsel) {
        select_rows(p, bh, t, smem);
    } else {
        if (p.v_in_logits)
            wait_count(p, p.ncand + (size_t)bh * kCandStride + 2, (uint32_t)v_direct_groups(nb, HD));
        lowres_rows<HD>(p, bh, (t - nsel) * kLoRows, smem);
    }
}

// ---------------------------------------------------------------- BigBird layout
// A static block-sparse pattern as a selection of 32-token blocks, for the
// same attention and join kernels ([BigBird]: a window of three blocks, two
// global blocks and num_random_blocks random blocks per query block).  With
// pattern blocks of bs = 32 f tokens, nbb = N / bs, pattern row I attends
// pattern block J when I or J is the first or last block, |I - J| <= 1, or J
// is one of the row's given picks (picks outside [0, nbb) name nothing; a
// block named twice is attended once); a pattern cell is f x f cells of
// 32-token blocks.  One workgroup per head (on the head's XCD); it also
// writes the blocks' mask words and counts, which pooling writes on the MRA
// path.
__global__ __launch_bounds__(kSelThreads) void bigbird_layout_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb, words = p.words;
    const int bh = blockIdx.x;
    if (bh >= p.BH) return;
    const int b = bh / p.H, tid = threadIdx.x;
    // the device error word starts clear (pooling clears it on the MRA path);
    // this kernel cannot set a bit of its own, since the stream is sized for
    // the pattern's largest count, so the attention kernel's bits stay exact
    if (bh == 0 && tid == 0) {
        p.error[0] = 0;
        p.error[1] = p.save_stats;
    }
    const SelectLds L = select_lds(nb);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + L.bitmap);
    int* rc = reinterpret_cast<int*>(smem + L.rc);
    int* ic = reinterpret_cast<int*>(smem + L.ic);
    uint32_t* mbv = reinterpret_cast<uint32_t*>(smem + L.mbv);
    uint64_t* scan64 = reinterpret_cast<uint64_t*>(smem + L.scan);
    const int f = p.bb_f, nbb = nb / f, r = p.bb_r;
    if (tid < nb) {
        // block tid's mask word: bit t = token 32 tid + t is valid
        uint32_t m = 0xFFFFFFFFu;
        if (p.mask) {
            const uint4* src = reinterpret_cast<const uint4*>(p.mask + (size_t)b * p.N + (size_t)tid * kBlock);
            m = 0u;
#pragma unroll
            for (int x = 0; x < 2; x++) {
                const uint4 u = src[x];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int y = 0; y < 16; y++)
                    if ((w4[y >> 2] >> (8 * (y & 3))) & 0xFFu) m |= 1u << (16 * x + y);
            }
        }
        mbv[tid] = m;
        if (bh % p.H == 0) {
            p.mbits[(size_t)b * nb + tid] = m;
            p.cnt[(size_t)b * nb + tid] = __popc(m);
        }
        // row tid of the bitmap belongs to this thread alone
        uint32_t* row = bitmap + (size_t)tid * words;
        for (int w = 0; w < words; w++) row[w] = 0u;
        const int I = tid / f;
        auto attend = [&](int J) {
            for (int c = 0; c < f; c++) {
                const int j = f * J + c;
                row[j >> 5] |= 1u << (j & 31);
            }
        };
        if (I == 0 || I == nbb - 1) {
            for (int w = 0; w < words; w++) row[w] = (w + 1) * 32 <= nb ? 0xFFFFFFFFu : (1u << (nb & 31)) - 1u;
        } else {
            attend(0);
            attend(nbb - 1);
            for (int J = I - 1; J <= I + 1; J++) attend(J);
            const int32_t* picks = p.bb_rand + ((size_t)bh * nbb + I) * r;
            for (int x = 0; x < r; x++) {
                const int J = picks[x];
                if (J >= 0 && J < nbb) attend(J);
            }
        }
    }
    // the word counts go where the selector keeps its histogram
    emit_stream(p, bh, bitmap, mbv, rc, ic, scan64, reinterpret_cast<uint16_t*>(smem + L.hist), -1);
}

}  // namespace

template <bool kGiven, int HD>
static hipError_t launch_logits_t(const Params& p, hipStream_t s) {
    if (fused_select(p.BH, p.nb, p.d, p.mode)) return hipSuccess;   // lgsel_kernel forms the logits
    const int tiles_per_head = (p.nb + kRT - 1) / kRT;
    static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&logits_kernel<kGiven, HD>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a1 != hipSuccess) return a1;
    const int heads_per_xcd = (p.BH + 7) / 8;
    int grid = 8 * heads_per_xcd * tiles_per_head;
    size_t lds = logits_lds(p.nb, HD).total;
    if (!kGiven && p.v_in_logits) {
        grid += 8 * heads_per_xcd * v_groups_per_head(p.nb, p.dtype, HD);
        if (lds < (size_t)kVUnitsPerGroup * kVUnitBytes) lds = (size_t)kVUnitsPerGroup * kVUnitBytes;
    }
    hipLaunchKernelGGL((logits_kernel<kGiven, HD>), dim3(grid), dim3(kLgThreads), lds, s, p);
    return hipGetLastError();
}

// Whether the logits launch pools V: full mode, and its logits workgroups
// at most one per CU of the device, so that the V workgroups run beside them.
bool v_pooled_in_logits(int mode, int BH, int nb, int d) {
    if (mode != 0) return false;
    if (fused_select(BH, nb, d, mode)) return true;   // lgsel_kernel: V workgroups after the logits ones
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return false;
        cus[dev] = n;
    }
    return 8 * ((BH + 7) / 8) * ((nb + kRT - 1) / kRT) <= cus[dev];
}

hipError_t launch_logits(const Params& p, hipStream_t s) {
    return p.d == 128 ? launch_logits_t<false, 128>(p, s) : launch_logits_t<false, 64>(p, s);
}
hipError_t launch_logits_given(const Params& p, hipStream_t s) {
    return p.d == 128 ? launch_logits_t<true, 128>(p, s) : launch_logits_t<true, 64>(p, s);
}

hipError_t launch_premark(const Params& p, hipStream_t s) {
    if (!premarked(p.nb)) return hipSuccess;
    const uint32_t ncell = (uint32_t)p.nb * (uint32_t)p.nb;
    const int ntiles = (int)((ncell + kTileCells - 1) / kTileCells);
    const int heads_per_xcd = (p.BH + 7) / 8;
    hipLaunchKernelGGL(premark_kernel, dim3(8 * heads_per_xcd * ntiles), dim3(kSelThreads), 0, s, p);
    return hipGetLastError();
}

template <int HD>
static size_t lgsel_lds(int nb, int mode) {
    size_t lds = fused_logits_lds(HD);
    if (tile_lds(nb).total > lds) lds = tile_lds(nb).total;
    if (mode == 0 && lowres_lds(nb, HD) > lds) lds = lowres_lds(nb, HD);
    return lds;
}

template <bool kGiven, int HD>
static hipError_t launch_lgsel_t(const Params& p, hipStream_t s) {
    static const hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void*>(&lgsel_kernel<kGiven, HD>),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a != hipSuccess) return a;
    const size_t lds = lgsel_lds<HD>(p.nb, p.mode);
    const int heads_per_xcd = (p.BH + 7) / 8;
    int grid = 8 * heads_per_xcd * (p.nb / kFusedRows);
    if (!kGiven && p.v_in_logits) grid += 8 * heads_per_xcd * v_direct_groups(p.nb, HD);
    hipLaunchKernelGGL((lgsel_kernel<kGiven, HD>), dim3(grid), dim3(kSelThreads), lds, s, p);
    return hipGetLastError();
}

// Whether heads of nb block rows take the one-launch logits and selection:
// heads of 64 or 128 block rows, and every logits workgroup of the launch
// resident on the device at once (its occupancy times the CU count).  The
// workgroups of a head wait for one another, and the low-res ones for the V
// workgroups after all logits workgroups; with every logits workgroup
// resident, the V workgroups get the CUs that the logits-only and selecting
// workgroups free, so every wait ends.  Larger grids take the separate
// logits and selection launches.
bool fused_select(int BH, int nb, int d, int mode) {
    if (!row_tiled(nb) || (d != 64 && d != 128)) return false;
    static int cap[64][2][2] = {};   // resident workgroups per device, head size and mode
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    int& c = cap[dev][d == 128][mode == 0];
    if (c == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return false;
        // the LDS of the larger head size of rows (128) bounds both
        const hipError_t e =
            d == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &per_cu, reinterpret_cast<const void*>(&lgsel_kernel<false, 128>), kSelThreads,
                           lgsel_lds<128>(128, mode))
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &per_cu, reinterpret_cast<const void*>(&lgsel_kernel<false, 64>), kSelThreads,
                           lgsel_lds<64>(128, mode));
        if (e != hipSuccess || per_cu <= 0) return false;
        c = per_cu * cus;
    }
    return 8 * ((BH + 7) / 8) * (nb / kFusedRows) <= c;
}

hipError_t launch_select(const Params& p, hipStream_t s) {
    if (fused_select(p.BH, p.nb, p.d, p.mode)) {
        if (p.logits_given) return p.d == 128 ? launch_lgsel_t<true, 128>(p, s) : launch_lgsel_t<true, 64>(p, s);
        return p.d == 128 ? launch_lgsel_t<false, 128>(p, s) : launch_lgsel_t<false, 64>(p, s);
    }
    static const hipError_t a2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a2 != hipSuccess) return a2;
    const int bh_pad = 8 * ((p.BH + 7) / 8);
    const int lowres_wgs = p.mode == 0 ? bh_pad * ((p.nb + kLoRows - 1) / kLoRows) : 0;
    size_t lds = select_lds(p.nb).total;
    if (p.mode == 0 && lowres_lds(p.nb, p.d) > lds) lds = lowres_lds(p.nb, p.d);
    hipLaunchKernelGGL(select_kernel, dim3(bh_pad + lowres_wgs), dim3(kSelThreads), lds, s, p);
    return hipGetLastError();
}

}  // namespace mra

namespace mra {
hipError_t launch_bigbird_layout(const Params& p, hipStream_t s) {
    static const hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void*>(&bigbird_layout_kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a != hipSuccess) return a;
    hipLaunchKernelGGL(bigbird_layout_kernel, dim3(p.BH), dim3(kSelThreads), select_lds(p.nb).total, s, p);
    return hipGetLastError();
}
}  // namespace mra
