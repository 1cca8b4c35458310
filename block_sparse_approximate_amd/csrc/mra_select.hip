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
//     block, rows cut into segments of at most kChunk blocks.
// A thread holds 16 cell keys in registers (the whole head up to N = 4096;
// longer heads are walked in tiles of 16384 cells with the next tile in
// flight), and wave w's cells of a tile are 64 consecutive cells, so one
// ballot is 64 consecutive bits of the selection.
//
// premark_kernel: for heads longer than one tile (with nb a multiple of 64)
// the marking pass runs before the selector, one workgroup per tile, so the
// selector only loads the bitmap of sure cells and the candidate list.
// The kernels are separate launches: the kernel boundary is what makes one
// workgroup's output visible to another, with no device-wide fences.
// The translation unit is built with -ffp-contract=off so that every fp32
// operation is the one written.
#include "mra_common.h"

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

// Rows of the low-res weight tile: nb + 4 floats (the pad spreads the rows
// over the LDS banks for the MFMA operand reads).
__host__ __device__ inline int wl_stride(int nb) { return nb + 4; }

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

// ---------------------------------------------------------------- helpers
// Exclusive scan of one value per thread over the select workgroup.
// Returns the exclusive prefix; *total gets the sum.  Uses scan[kSelWaves + 1].
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* scan, T* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) scan[wave] = x;
    __syncthreads();
    if (threadIdx.x < 64) {
        const T t = threadIdx.x < kSelWaves ? scan[threadIdx.x] : T(0);
        T y = t;
#pragma unroll
        for (int off = 1; off < kSelWaves; off <<= 1) {
            const T z = __shfl_up(y, off, 64);
            if ((int)threadIdx.x >= off) y += z;
        }
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
    uint32_t x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    const uint32_t above = x - local;
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
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
    const bool raw = p.rank_raw != 0;
#pragma unroll
    for (int t = 0; t < kMaxColTiles; t++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int i = q < 2 ? ra : rb, j = t * kCT + lane + 64 * (q & 1);
            if (t < ntile && i < nb && j < nb) {
                const float sv = sc[t][q];
                if (!kGiven) Sg[(size_t)i * nb + j] = sv;
                const int cjq = (q & 1) ? cj[t].y : cj[t].x;
                const float s = cell_score(sv, q < 2 ? ma : mb, i, j, (q < 2 ? cia : cib) > 0, cjq > 0, pf, pd, raw);
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
// Full mode, [MRA] "第四步": the low-resolution attention of 32 block rows of
// head bh over every key block, selected or not,
//   lo_all_i = sum_j w_ij vhat_j,  ll_all_i = sum_j w_ij,  w_ij = cnt_j exp(S_ij - m_i),
// from which the block attention later takes the selected cells back out.
// These workgroups ride in the selector's launch: they need only the logits
// kernel's output, so they run on the CUs the per-head selectors leave idle.
// The product runs on v_mfma_f32_16x16x4f32: wave w takes the 16-row tile
// w / 8, the 16-channel tile (w / 2) % 4 and the key half w % 2 of each key
// tile; A lane l holds W[l % 16][k = l / 16], B lane l holds
// vhat[k = l / 16][l % 16], and accumulator e of lane l is row 4 (l / 16) + e,
// channel l % 16.
constexpr int kLoRows = 32;
// key blocks per staged vhat tile: 128 for 64-channel heads, 64 for 128
__host__ __device__ constexpr int lowres_keys(int hd) { return hd == 64 ? kCT : kCT / 2; }

__host__ __device__ inline size_t lowres_lds(int nb, int hd) {
    return align16((size_t)kLoRows * wl_stride(nb) * 4) + align16((size_t)lowres_keys(hd) * hat_stride(hd) * 4) +
           align16(2 * 8 * 64 * 4 * 4);
}

template <int HD>
__device__ __forceinline__ void lowres_rows(const Params& p, int bh, int row0, unsigned char* smem) {
    constexpr int kVtStride = hat_stride(HD);
    constexpr int kKT = lowres_keys(HD);     // key blocks per vhat tile
    constexpr int kCTW = HD / 64;            // 16-channel tiles per wave
    const int nb = p.nb, nbp = wl_stride(nb);
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float* wl = reinterpret_cast<float*>(smem);
    float* vt = reinterpret_cast<float*>(smem + align16((size_t)kLoRows * nbp * 4));
    float* red = vt + align16((size_t)kKT * kVtStride * 4) / 4;
    const float* S = p.logits + (size_t)bh * nb * nb;
    const float* vh = p.vhat + (size_t)bh * nb * HD;
    const int* cnt = p.cnt + (size_t)b * nb;
    constexpr int kVLoads = kKT * (HD / 4) / kSelThreads;   // float4s of one vhat tile per thread

    // vhat tile 0 in flight first; the weights: wave w owns rows 2w, 2w + 1
    float4 vv[kVLoads];
#pragma unroll
    for (int e = 0; e < kVLoads; e++) {
        const int x = tid + e * kSelThreads, j = x / (HD / 4);
        vv[e] = j < nb ? *reinterpret_cast<const float4*>(vh + (size_t)j * HD + (x % (HD / 4)) * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    constexpr int kJ = kMaxColTiles * kCT / 64;   // key blocks per lane (nb <= 512)
    const int ia = row0 + 2 * wave, ib = ia + 1;   // this wave's two rows
    float sa[kJ], sb[kJ];
    int cv[kJ];
#pragma unroll
    for (int t = 0; t < kJ; t++) {
        const int j = lane + 64 * t;
        cv[t] = j < nb ? cnt[j] : 0;
        sa[t] = (ia < nb && j < nb) ? S[(size_t)ia * nb + j] : 0.f;
        sb[t] = (ib < nb && j < nb) ? S[(size_t)ib * nb + j] : 0.f;
    }
    const float ma = ia < nb ? p.rowmax[(size_t)bh * nb + ia] : 0.f;
    const float mb = ib < nb ? p.rowmax[(size_t)bh * nb + ib] : 0.f;
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int t = 0; t < kJ; t++) {
        const int j = lane + 64 * t;
        if (j < nb) {
            const float wa = ia < nb ? lowres_weight(sa[t], ma, cv[t]) : 0.f;
            const float wb = ib < nb ? lowres_weight(sb[t], mb, cv[t]) : 0.f;
            wl[(2 * wave) * nbp + j] = wa;
            wl[(2 * wave + 1) * nbp + j] = wb;
            la += wa;
            lb += wb;
        }
    }
    la = wave_sum(la);
    lb = wave_sum(lb);
    if (lane == 0) {
        if (ia < nb) p.ll_all[(size_t)bh * nb + ia] = la;
        if (ib < nb) p.ll_all[(size_t)bh * nb + ib] = lb;
    }
    // wave w: row tile w / 8, 16-channel tiles c = (w / 2) % 4 + 4 x (x < HD / 64),
    // key half w % 2
    const int rt = wave >> 3, ct = (wave >> 1) & 3, kh2 = wave & 1;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 acc[kCTW];
#pragma unroll
    for (int x = 0; x < kCTW; x++) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < nb; j0 += kKT) {
        __syncthreads();   // the weights are in place; every wave is done with the previous tile
#pragma unroll
        for (int e = 0; e < kVLoads; e++) {
            const int x = tid + e * kSelThreads;
            *reinterpret_cast<float4*>(vt + (x / (HD / 4)) * kVtStride + (x % (HD / 4)) * 4) = vv[e];
        }
        __syncthreads();
        if (j0 + kKT < nb) {
#pragma unroll
            for (int e = 0; e < kVLoads; e++) {
                const int x = tid + e * kSelThreads, j = j0 + kKT + x / (HD / 4);
                vv[e] = j < nb ? *reinterpret_cast<const float4*>(vh + (size_t)j * HD + (x % (HD / 4)) * 4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        const int jn = min(kKT, nb - j0);
#pragma unroll
        for (int k4 = 0; k4 < kKT / 2; k4 += 4) {
            const int k = kh2 * (kKT / 2) + k4 + (lane >> 4);
            const bool ok = k < jn;
            const float a = ok ? wl[(rt * 16 + (lane & 15)) * nbp + j0 + k] : 0.f;
#pragma unroll
            for (int x = 0; x < kCTW; x++) {
                const float bv = ok ? vt[k * kVtStride + (ct + 4 * x) * 16 + (lane & 15)] : 0.f;
                acc[x] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc[x], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int x = 0; x < kCTW; x++) {
        const int tile = rt * 4 + ct + 8 * x;   // 0 .. 8 kCTW - 1
        if (kh2 == 1) *reinterpret_cast<f32x4*>(red + (tile * 64 + lane) * 4) = acc[x];
    }
    __syncthreads();
    if (kh2 == 0) {
#pragma unroll
        for (int x = 0; x < kCTW; x++) {
            const int tile = rt * 4 + ct + 8 * x;
            const f32x4 o = *reinterpret_cast<const f32x4*>(red + (tile * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int row = row0 + rt * 16 + 4 * (lane >> 4) + e;
                if (row < nb)
                    p.lo_all[((size_t)bh * nb + row) * HD + (ct + 4 * x) * 16 + (lane & 15)] = acc[x][e] + o[e];
            }
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
// words in LDS (written before the call; read after its barriers).  expect:
// the number of selected cells the caller made (the error word's bit 2
// flags another count), or -1 when the count is the layout's own (it must
// stay within the stream's capacity p.K).  Called by a whole kSelThreads
// workgroup.
__device__ __forceinline__ void emit_stream(const Params& p, int bh, const uint32_t* bitmap, const uint32_t* mbv, int* rc,
                            int* ic, uint64_t* scan64, int64_t expect) {
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
            for (int w = 0; w < words; w++) c += __popc(bitmap[i * words + w]);
        const int it = (c + kChunk - 1) / kChunk;
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
    // column lists and the attention stream records: one thread per selected
    // cell e (CSR order).  Its block row is the last row whose start is at
    // most e; its key block is the bit of rank e - start among the set bits
    // of that row's bitmap.
    int32_t* col = p.col + (size_t)bh * p.K;
    BlkRec* recs = p.recs + (size_t)bh * p.K;
    const int tcap = (int)min((int64_t)rc[nb], p.K);
    for (int e = tid; e < tcap; e += kSelThreads) {
        int lo = 0, hi = nb - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (rc[mid] <= e) lo = mid;
            else hi = mid - 1;
        }
        const int i = lo, o = rc[i], n = rc[i + 1] - o, rank = e - o;
        // the word that holds the cell, then the bit: halve the word five
        // times, keeping the half that holds the remaining rank
        const uint32_t* row = bitmap + i * words;
        int r = rank, w = 0;
        uint32_t bits = row[0];
        int c = __popc(bits);
        while (r >= c && w + 1 < words) {
            r -= c;
            bits = row[++w];
            c = __popc(bits);
        }
        int pos = 0;
#pragma unroll
        for (int half = 16; half > 0; half >>= 1) {
            const uint32_t low = bits & ((1u << half) - 1u);
            const int cl = __popc(low);
            if (r >= cl) {
                r -= cl;
                bits >>= half;
                pos += half;
            } else {
                bits = low;
            }
        }
        const int j = w * 32 + pos;
        col[e] = j;
        const int nit = (n + kChunk - 1) / kChunk, sg = rank / kChunk;
        const int len = min(kChunk, n - sg * kChunk);
        recs[e] = BlkRec{rec_ij(i, j), mbv[j], 0u, rec_info(ic[i] + sg, rank - sg * kChunk, len, nit == 1)};
    }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb;
    // workgroups [0, BH_pad) select, one per head (BH_pad = BH rounded up to
    // a multiple of 8, so workgroup bh runs on XCD bh % 8); in full mode the
    // rest sum the low-res attention of 32 rows each, placed on the XCD of
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
    emit_stream(p, bh, bitmap, mbv, rc, ic, scan64, p.K);
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
    if (bh == 0 && tid == 0) *p.error = 0;
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
    emit_stream(p, bh, bitmap, mbv, rc, ic, scan64, -1);
}

}  // namespace

template <bool kGiven, int HD>
static hipError_t launch_logits_t(const Params& p, hipStream_t s) {
    const int tiles_per_head = (p.nb + kRT - 1) / kRT;
    static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&logits_kernel<kGiven, HD>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a1 != hipSuccess) return a1;
    const int heads_per_xcd = (p.BH + 7) / 8;
    hipLaunchKernelGGL((logits_kernel<kGiven, HD>), dim3(8 * heads_per_xcd * tiles_per_head), dim3(kLgThreads),
                       logits_lds(p.nb, HD).total, s, p);
    return hipGetLastError();
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

hipError_t launch_select(const Params& p, hipStream_t s) {
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
