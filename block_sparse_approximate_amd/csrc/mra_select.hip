// mra_select.hip — step 1 low-resolution logits and step 2 block selection
// ([MRA] "第一步" and "第二步").
//
// logits_kernel: workgroup (bh, t) computes the logits of 16 block rows of
// head bh,  S_ij = fma-chain_c(qhat_i[c], khat_j[c]) * tau  (fp32, channels in
// order from +0, the canonical order), the row maximum over non-empty key
// blocks, the selection score of each cell and a 4096-bin histogram of the
// top 12 bits of its ordered key, which it adds into the head's histogram.
//
// select_kernel: one workgroup per head selects the top-K cells:
//   * the composite key of a cell is (ordered fp32 score, then the inverse
//     flat index), so all keys differ and "the first K cells in (score
//     descending, flat index ascending)" are exactly the K largest keys;
//   * a radix select walks the key from the top: the histogram fixes the
//     first 12 bits, further 12-bit passes run only while that bin holds
//     more than kCap cells; one pass then marks the cells above the bin as
//     selected and copies the cells inside it into LDS, where 8-bit passes
//     find the K-th largest key T;
//   * the selected set {key >= T} is written as a bitmap, as CSR (row_ptr,
//     col ascending) and as the attention stream: one record per selected
//     block, rows cut into segments of at most kChunk blocks.
// The scores of a head are staged through LDS in tiles of 16384 cells (the
// whole head up to N = 4096).  Every pass gives each thread a run of cells
// and issues all of a thread's global loads before their first use, so a
// pass costs about one memory round trip and no chain of LDS round trips.
// The two kernels are separate launches: the kernel boundary is what makes
// one workgroup's logits visible to another, with no device-wide fences.
// The translation unit is built with -ffp-contract=off so that every fp32
// operation is the one written.
#include "mra_common.h"

namespace mra {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRT = 16;        // block rows per logits workgroup
constexpr int kCT = 128;       // key blocks per logits tile
constexpr int kCap = 4096;     // selection candidates held in LDS
constexpr int kTile = 16384;   // score cells staged in LDS at a time
constexpr int kRun = kTile / kThreads;   // cells per thread and tile

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// ---------------------------------------------------------------- LDS plans
struct LogitsLds {
    size_t qT, kT, srow, cntv, hist, small, total;
};

__host__ __device__ inline LogitsLds logits_lds(int nb) {
    LogitsLds L;
    size_t o = 0;
    L.qT = o; o = align16(o + 64 * kRT * 4);
    L.kT = o; o = align16(o + 64 * kCT * 4);
    L.srow = o; o = align16(o + (size_t)kRT * nb * 4);
    L.cntv = o; o = align16(o + (size_t)nb * 4);
    L.hist = o; o = align16(o + kHistBins * 4);
    L.small = o; o = align16(o + 64 * 4);
    L.total = o;
    return L;
}

// Rows of scores staged in LDS at a time by the selector.
__host__ __device__ inline int tile_rows(int nb) {
    const int r = kTile / nb;
    return r < 1 ? 1 : (r > nb ? nb : r);
}

struct SelectLds {
    size_t tile, hist, cand, bitmap, rm, cntv, rc, ic, mbv, scan, small, total;
};

__host__ __device__ inline SelectLds select_lds(int nb) {
    SelectLds L;
    const int words = (nb + 31) / 32;
    size_t o = 0;
    L.tile = o; o = align16(o + (size_t)tile_rows(nb) * nb * 4);
    L.hist = o; o = align16(o + kHistBins * 4);
    L.cand = o; o = align16(o + (size_t)kCap * 8);
    L.bitmap = o; o = align16(o + (size_t)nb * words * 4);
    L.rm = o; o = align16(o + (size_t)nb * 4);
    L.cntv = o; o = align16(o + (size_t)nb * 4);
    L.rc = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.ic = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.mbv = o; o = align16(o + (size_t)nb * 4);
    L.scan = o; o = align16(o + 64 * 4);
    L.small = o; o = align16(o + 64 * 8);
    L.total = o;
    return L;
}

// ---------------------------------------------------------------- helpers
// Exclusive scan of one int per thread over the workgroup (kThreads).
// Returns the exclusive prefix; *total gets the sum.  Uses scan[kWaves + 1].
__device__ int block_excl_scan(int v, int* scan, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) scan[wave] = x;
    __syncthreads();
    if (threadIdx.x < 64) {
        const int t = threadIdx.x < kWaves ? scan[threadIdx.x] : 0;
        int y = t;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            int z = __shfl_up(y, off, 64);
            if ((int)threadIdx.x >= off) y += z;
        }
        if (threadIdx.x < kWaves) scan[threadIdx.x] = y - t;
        if (threadIdx.x == kWaves - 1) scan[kWaves] = y;
    }
    __syncthreads();
    const int ex = scan[wave] + x - v;
    *total = scan[kWaves];
    __syncthreads();
    return ex;
}

struct BinPick {
    uint32_t bin, above, count;
};

// Find, in a histogram of kHistBins bins held in LDS, the bin where the
// count taken from the top first reaches `need`.  Each thread owns 8 bins.
__device__ BinPick pick_bin(const uint32_t* h, uint32_t need, int* scan, uint32_t* small) {
    const int rt = kThreads - 1 - (int)threadIdx.x;   // reversed: the top bins come first
    uint32_t local = 0;
#pragma unroll
    for (int e = 0; e < 8; e++) local += h[rt * 8 + e];
    int tot;
    const uint32_t above = (uint32_t)block_excl_scan((int)local, scan, &tot);
    if (above < need && need <= above + local) {
        uint32_t acc = above;
        for (int e = 7; e >= 0; e--) {
            const uint32_t c = h[rt * 8 + e];
            if (acc + c >= need) {
                small[0] = (uint32_t)(rt * 8 + e);
                small[1] = acc;
                small[2] = c;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
    BinPick r{small[0], small[1], small[2]};
    __syncthreads();
    return r;
}

__device__ __forceinline__ uint64_t tile_key(float logit, const float* rm, const int* cntv, int nb, int i, int j,
                                            int pf, int pd) {
    const float s = cell_score(logit, rm[i], i, j, cntv[i] > 0, cntv[j] > 0, pf, pd);
    return cell_key64(float_key(s), (uint32_t)(i * nb + j));
}

// Global loads of a tile of scores into registers (all issued at once).
__device__ __forceinline__ void fetch_tile(const float* __restrict__ S, int r0, int rows, int nb, float (&v)[kRun]) {
    const int n = rows * nb;
    const float* src = S + (size_t)r0 * nb;
#pragma unroll
    for (int e = 0; e < kRun; e++) {
        const int x = threadIdx.x + e * kThreads;
        v[e] = x < n ? src[x] : 0.0f;
    }
}

__device__ __forceinline__ void store_tile(int rows, int nb, const float (&v)[kRun], float* tile) {
    const int n = rows * nb;
#pragma unroll
    for (int e = 0; e < kRun; e++) {
        const int x = threadIdx.x + e * kThreads;
        if (x < n) tile[x] = v[e];
    }
}

// ---------------------------------------------------------------- logits
// kGiven: the logits are already in p.logits (selector hook); skip their
// computation and only form row maxima and the histogram.
template <bool kGiven>
__global__ __launch_bounds__(kThreads) void logits_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb;
    const int tiles_per_head = (nb + kRT - 1) / kRT;
    const int bh = blockIdx.x / tiles_per_head;
    const int row0 = (blockIdx.x - bh * tiles_per_head) * kRT;
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float tau = (float)(1.0 / __builtin_sqrt((double)p.d));

    const LogitsLds L = logits_lds(nb);
    float* qT = reinterpret_cast<float*>(smem + L.qT);
    float* kT = reinterpret_cast<float*>(smem + L.kT);
    float* srow = reinterpret_cast<float*>(smem + L.srow);
    int* cntv = reinterpret_cast<int*>(smem + L.cntv);
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    float* rmax = reinterpret_cast<float*>(smem + L.small);
    const float* qh = p.qhat + (size_t)bh * nb * kHeadDim;
    const float* kh = p.khat + (size_t)bh * nb * kHeadDim;

    // every global load of the prologue first, then the LDS stores
    constexpr int kKLoads = kCT * (kHeadDim / 4) / kThreads;   // float4s of one khat tile per thread
    int cn = tid < nb ? p.cnt[b * nb + tid] : 0;               // nb <= 512 = kThreads
    float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 kv[kKLoads];
    if (!kGiven) {
        if (tid < kRT * kHeadDim / 4) {
            const int r = tid / (kHeadDim / 4), c4 = (tid % (kHeadDim / 4)) * 4;
            if (row0 + r < nb) qv = *reinterpret_cast<const float4*>(qh + (size_t)(row0 + r) * kHeadDim + c4);
        }
#pragma unroll
        for (int e = 0; e < kKLoads; e++) {
            const int x = tid + e * kThreads, jj = x % kCT, c4 = (x / kCT) * 4;
            kv[e] = jj < nb ? *reinterpret_cast<const float4*>(kh + (size_t)jj * kHeadDim + c4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        for (int x = tid; x < kRT * nb; x += kThreads) {
            const int r = x / nb, j = x - r * nb;
            srow[x] = (row0 + r < nb) ? p.logits[((size_t)bh * nb + row0 + r) * nb + j] : 0.0f;
        }
    }
    if (tid < nb) cntv[tid] = cn;
    for (int x = tid; x < kHistBins; x += kThreads) hist[x] = 0u;
    if (!kGiven && tid < kRT * kHeadDim / 4) {
        const int r = tid / (kHeadDim / 4), c4 = (tid % (kHeadDim / 4)) * 4;
        qT[(c4 + 0) * kRT + r] = qv.x;
        qT[(c4 + 1) * kRT + r] = qv.y;
        qT[(c4 + 2) * kRT + r] = qv.z;
        qT[(c4 + 3) * kRT + r] = qv.w;
    }
    const int r0 = 2 * wave;          // this wave's two block rows
    for (int j0 = 0; j0 < (kGiven ? 0 : nb); j0 += kCT) {
        __syncthreads();
        // kT[c][jj] = khat[j0 + jj][c]
#pragma unroll
        for (int e = 0; e < kKLoads; e++) {
            const int x = tid + e * kThreads, jj = x % kCT, c4 = (x / kCT) * 4;
            kT[(c4 + 0) * kCT + jj] = kv[e].x;
            kT[(c4 + 1) * kCT + jj] = kv[e].y;
            kT[(c4 + 2) * kCT + jj] = kv[e].z;
            kT[(c4 + 3) * kCT + jj] = kv[e].w;
        }
        __syncthreads();
        if (j0 + kCT < nb) {   // the next khat tile is in flight during this one
#pragma unroll
            for (int e = 0; e < kKLoads; e++) {
                const int x = tid + e * kThreads, jj = x % kCT, c4 = (x / kCT) * 4;
                kv[e] = j0 + kCT + jj < nb
                            ? *reinterpret_cast<const float4*>(kh + (size_t)(j0 + kCT + jj) * kHeadDim + c4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
#pragma unroll 8
        for (int c = 0; c < kHeadDim; c++) {
            const float2 q2 = *reinterpret_cast<const float2*>(qT + c * kRT + r0);
            const float2 k2 = *reinterpret_cast<const float2*>(kT + c * kCT + 2 * lane);
            a00 = __builtin_fmaf(q2.x, k2.x, a00);
            a01 = __builtin_fmaf(q2.x, k2.y, a01);
            a10 = __builtin_fmaf(q2.y, k2.x, a10);
            a11 = __builtin_fmaf(q2.y, k2.y, a11);
        }
        const int j = j0 + 2 * lane;
        if (j < nb) {
            srow[(size_t)r0 * nb + j] = a00 * tau;
            srow[(size_t)(r0 + 1) * nb + j] = a10 * tau;
        }
        if (j + 1 < nb) {
            srow[(size_t)r0 * nb + j + 1] = a01 * tau;
            srow[(size_t)(r0 + 1) * nb + j + 1] = a11 * tau;
        }
    }
    __syncthreads();
    // row maxima over non-empty key blocks (exact: max does not round)
    for (int rr = 0; rr < 2; rr++) {
        const int r = r0 + rr;
        float m = -__builtin_inff();
        for (int j = lane; j < nb; j += 64)
            if (cntv[j] > 0) m = fmaxf(m, srow[(size_t)r * nb + j]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        if (lane == 0) rmax[r] = m;
    }
    __syncthreads();
    // scores -> histogram of the top 12 key bits; logits and maxima out
    float* Sg = p.logits + (size_t)bh * nb * nb;
    for (int x = tid; x < kRT * nb; x += kThreads) {
        const int r = x / nb, j = x - r * nb, i = row0 + r;
        if (i >= nb) continue;
        const float sv = srow[x];
        if (!kGiven) Sg[(size_t)i * nb + j] = sv;
        const float s = cell_score(sv, rmax[r], i, j, cntv[i] > 0, cntv[j] > 0, p.prior_first, p.prior_diag);
        atomicAdd(&hist[float_key(s) >> (32 - kHistBits)], 1u);
    }
    for (int r = tid; r < kRT; r += kThreads)
        if (row0 + r < nb) p.rowmax[(size_t)bh * nb + row0 + r] = rmax[r];
    __syncthreads();
    uint32_t* gh = p.hist + (size_t)bh * kHistBins;
    for (int x = tid; x < kHistBins; x += kThreads)
        if (hist[x]) atomicAdd(&gh[x], hist[x]);
}

// ---------------------------------------------------------------- select
__global__ __launch_bounds__(kThreads) void select_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb;
    const int bh = blockIdx.x;
    const int b = bh / p.H;
    const int tid = threadIdx.x;
    const SelectLds L = select_lds(nb);
    const int words = p.words;
    float* stile = reinterpret_cast<float*>(smem + L.tile);
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    uint64_t* cand = reinterpret_cast<uint64_t*>(smem + L.cand);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + L.bitmap);
    float* rm = reinterpret_cast<float*>(smem + L.rm);
    int* cntv = reinterpret_cast<int*>(smem + L.cntv);
    int* rc = reinterpret_cast<int*>(smem + L.rc);
    int* ic = reinterpret_cast<int*>(smem + L.ic);
    uint32_t* mbv = reinterpret_cast<uint32_t*>(smem + L.mbv);
    int* scan = reinterpret_cast<int*>(smem + L.scan);
    uint32_t* small = reinterpret_cast<uint32_t*>(smem + L.small);
    const float* S = p.logits + (size_t)bh * nb * nb;
    const int pf = p.prior_first, pd = p.prior_diag;
    const int trows = tile_rows(nb);
    const bool resident = trows >= nb;   // the whole head fits one tile: stage it once

    // prologue: all global loads, then the LDS stores
    {
        uint32_t hv[kHistBins / kThreads];
#pragma unroll
        for (int e = 0; e < kHistBins / kThreads; e++) hv[e] = p.hist[(size_t)bh * kHistBins + tid + e * kThreads];
        float tv[kRun];
        if (resident) fetch_tile(S, 0, nb, nb, tv);
        const int cn = tid < nb ? p.cnt[b * nb + tid] : 0;   // nb <= 512 = kThreads
        const float rv = tid < nb ? p.rowmax[(size_t)bh * nb + tid] : 0.f;
        const uint32_t mv = tid < nb ? p.mbits[b * nb + tid] : 0u;
        if (tid < nb) {
            cntv[tid] = cn;
            rm[tid] = rv;
            mbv[tid] = mv;
        }
#pragma unroll
        for (int e = 0; e < kHistBins / kThreads; e++) hist[tid + e * kThreads] = hv[e];
        for (int x = tid; x < nb * words; x += kThreads) bitmap[x] = 0u;
        if (resident) store_tile(nb, nb, tv, stile);
    }
    __syncthreads();

    uint32_t need = (uint32_t)p.K;
    BinPick bp = pick_bin(hist, need, scan, small);
    need -= bp.above;
    uint64_t prefix = bp.bin;
    int pbits = kHistBits;
    uint32_t count = bp.count;

    // further 12-bit passes while the bin is too large for LDS (tie-heavy inputs)
    while (count > (uint32_t)kCap && pbits < 64) {
        const int db = (64 - pbits) < 12 ? (64 - pbits) : 12;
        for (int x = tid; x < kHistBins; x += kThreads) hist[x] = 0u;
        for (int r0 = 0; r0 < nb; r0 += trows) {
            const int rows = min(trows, nb - r0);
            if (!resident) {
                float tv[kRun];
                fetch_tile(S, r0, rows, nb, tv);
                __syncthreads();
                store_tile(rows, nb, tv, stile);
            }
            __syncthreads();
            for (int x = tid; x < rows * nb; x += kThreads) {
                const int r = x / nb, j = x - r * nb, i = r0 + r;
                const uint64_t k64 = tile_key(stile[x], rm, cntv, nb, i, j, pf, pd);
                if ((k64 >> (64 - pbits)) == prefix)
                    atomicAdd(&hist[(uint32_t)((k64 >> (64 - pbits - db)) & ((1ull << db) - 1))], 1u);
            }
        }
        __syncthreads();
        bp = pick_bin(hist, need, scan, small);
        need -= bp.above;
        prefix = (prefix << db) | bp.bin;
        pbits += db;
        count = bp.count;
    }

    // One pass over the cells: cells above the bin are selected for sure
    // (bitmap), cells inside it are appended to the LDS candidate list.  A
    // wave takes 64 consecutive cells at a time, so its LDS reads are
    // conflict-free and, when a row holds a multiple of 64 blocks, one ballot
    // is two whole bitmap words.
    if (tid == 0) small[8] = 0u;
    const bool rows64 = (nb & 63) == 0;
    const int lane = tid & 63;
    for (int r0 = 0; r0 < nb; r0 += trows) {
        const int rows = min(trows, nb - r0);
        const int n = rows * nb;
        if (!resident) {
            float tv[kRun];
            fetch_tile(S, r0, rows, nb, tv);
            __syncthreads();
            store_tile(rows, nb, tv, stile);
        }
        __syncthreads();
        for (int x0 = tid - lane; x0 < n; x0 += kThreads) {
            const int x = x0 + lane;
            bool sure = false, hit = false;
            uint64_t k64 = 0;
            int i = 0, j = 0;
            if (x < n) {
                const int r = x / nb;
                j = x - r * nb;
                i = r0 + r;
                k64 = tile_key(stile[x], rm, cntv, nb, i, j, pf, pd);
                const uint64_t top = k64 >> (64 - pbits);
                sure = top > prefix;
                hit = top == prefix;
            }
            const uint64_t ms = __ballot(sure);
            if (rows64) {
                if (lane == 0) {
                    const int i0 = r0 + x0 / nb, j0 = x0 - (x0 / nb) * nb;
                    bitmap[i0 * words + (j0 >> 5)] = (uint32_t)ms;
                    bitmap[i0 * words + (j0 >> 5) + 1] = (uint32_t)(ms >> 32);
                }
            } else if (sure) {
                atomicOr(&bitmap[i * words + (j >> 5)], 1u << (j & 31));
            }
            const uint64_t mh = __ballot(hit);
            if (mh) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&small[8], (uint32_t)__popcll(mh));
                base = __shfl(base, 0, 64);
                if (hit) {
                    const uint32_t at = base + (uint32_t)__popcll(mh & ((1ull << lane) - 1ull));
                    if (at < (uint32_t)kCap) cand[at] = k64;
                }
            }
        }
    }
    __syncthreads();
    const uint32_t ncand_all = small[8];
    __syncthreads();
    const uint32_t ncand = ncand_all < (uint32_t)kCap ? ncand_all : (uint32_t)kCap;
    if (tid == 0 && ncand_all != count) atomicOr(reinterpret_cast<unsigned int*>(p.error), 1u);

    // 8-bit passes over the candidates until the K-th largest key is pinned down
    while (pbits < 64) {
        const int db = (64 - pbits) < 8 ? (64 - pbits) : 8;
        for (int x = tid; x < kHistBins; x += kThreads) hist[x] = 0u;
        __syncthreads();
        for (uint32_t c = tid; c < ncand; c += kThreads) {
            const uint64_t k64 = cand[c];
            if ((k64 >> (64 - pbits)) == prefix)
                atomicAdd(&hist[(uint32_t)((k64 >> (64 - pbits - db)) & ((1ull << db) - 1))], 1u);
        }
        __syncthreads();
        bp = pick_bin(hist, need, scan, small);
        need -= bp.above;
        prefix = (prefix << db) | bp.bin;
        pbits += db;
        if (bp.count == 1u && pbits < 64) {
            // a single cell left: it is the threshold
            for (uint32_t c = tid; c < ncand; c += kThreads) {
                if ((cand[c] >> (64 - pbits)) == prefix) {
                    small[10] = (uint32_t)(cand[c] >> 32);
                    small[11] = (uint32_t)cand[c];
                }
            }
            __syncthreads();
            prefix = ((uint64_t)small[10] << 32) | small[11];
            pbits = 64;
            __syncthreads();
        }
    }
    const uint64_t T = prefix;
    if (tid == 0) p.thresh[bh] = T;

    // candidates at or above the threshold join the bitmap
    for (uint32_t c = tid; c < ncand; c += kThreads) {
        const uint64_t k64 = cand[c];
        if (k64 >= T) {
            const uint32_t f = 0xFFFFFFFFu - (uint32_t)k64;
            const int i = (int)(f / (uint32_t)nb), j = (int)(f - (uint32_t)i * (uint32_t)nb);
            if (i < nb) atomicOr(&bitmap[i * words + (j >> 5)], 1u << (j & 31));
        }
    }
    __syncthreads();

    // CSR row pointers and segment (item) pointers
    int32_t* row_ptr = p.row_ptr + (size_t)bh * (nb + 1);
    int32_t* item_ptr = p.item_ptr + (size_t)bh * (nb + 1);
    int row_base = 0, item_base = 0;
    for (int i0 = 0; i0 < nb; i0 += kThreads) {
        const int i = i0 + tid;
        int c = 0;
        if (i < nb)
            for (int w = 0; w < words; w++) c += __popc(bitmap[i * words + w]);
        const int it = (c + kChunk - 1) / kChunk;
        int tc, ti;
        const int ec = block_excl_scan(c, scan, &tc);
        const int ei = block_excl_scan(it, scan, &ti);
        if (i < nb) {
            row_ptr[i] = row_base + ec;
            item_ptr[i] = item_base + ei;
            rc[i] = row_base + ec;
            ic[i] = item_base + ei;
        }
        row_base += tc;
        item_base += ti;
    }
    if (tid == 0) {
        row_ptr[nb] = row_base;
        item_ptr[nb] = item_base;
        rc[nb] = row_base;
        ic[nb] = item_base;
        small[12] = 0u;
        if ((int64_t)row_base != p.K || item_base > p.max_items) atomicOr(reinterpret_cast<unsigned int*>(p.error), 2u);
    }
    __syncthreads();

    // column lists and the attention stream records, one thread per row
    int32_t* col = p.col + (size_t)bh * p.K;
    BlkRec* recs = p.recs + (size_t)bh * p.K;
    uint32_t* gbits = p.selbits + (size_t)bh * nb * words;
    for (int x = tid; x < nb * words; x += kThreads) gbits[x] = bitmap[x];
    for (int i = tid; i < nb; i += kThreads) {
        const int o = rc[i], n = rc[i + 1] - o, first = ic[i];
        const int nit = (n + kChunk - 1) / kChunk;
        if (nit != 1) {   // no selected block, or several segments: the final kernel combines this row
            const uint32_t at = atomicAdd(&small[12], 1u);
            if (at < (uint32_t)nb) p.merge_rows[(size_t)bh * nb + at] = i;
        }
        int r = 0;
        for (int w = 0; w < words && r < n; w++) {
            uint32_t bits = bitmap[i * words + w];
            while (bits) {
                const int j = w * 32 + __builtin_ctz(bits);
                bits &= bits - 1;
                const int e = o + r;
                if (e < p.K) {
                    col[e] = j;
                    const int sg = r / kChunk;
                    const int len = min(kChunk, n - sg * kChunk);
                    recs[e] = BlkRec{i, j, mbv[j], rec_info(first + sg, r - sg * kChunk, len, nit == 1)};
                }
                r++;
            }
        }
    }
    __syncthreads();
    if (tid == 0) p.n_merge[bh] = (int32_t)min(small[12], (uint32_t)nb);
}

}  // namespace

template <bool kGiven>
static hipError_t launch_logits_t(const Params& p, hipStream_t s) {
    const int tiles_per_head = (p.nb + kRT - 1) / kRT;
    static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&logits_kernel<kGiven>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a1 != hipSuccess) return a1;
    hipLaunchKernelGGL(logits_kernel<kGiven>, dim3(p.BH * tiles_per_head), dim3(kThreads), logits_lds(p.nb).total,
                       s, p);
    return hipGetLastError();
}

hipError_t launch_logits(const Params& p, hipStream_t s) { return launch_logits_t<false>(p, s); }
hipError_t launch_logits_given(const Params& p, hipStream_t s) { return launch_logits_t<true>(p, s); }

hipError_t launch_select(const Params& p, hipStream_t s) {
    static const hipError_t a2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (a2 != hipSuccess) return a2;
    hipLaunchKernelGGL(select_kernel, dim3(p.BH), dim3(kThreads), select_lds(p.nb).total, s, p);
    return hipGetLastError();
}

}  // namespace mra
