// mra_select.hip — step 1 low-resolution logits and step 2 block selection
// ([MRA] "第一步" and "第二步").
//
// One launch.  Workgroup (bh, t) computes the logits of 16 block rows of
// head bh:  S_ij = fma-chain_c(qhat_i[c], khat_j[c]) * tau  (fp32, channels in
// order from +0, the canonical order), the row maximum over non-empty key
// blocks, the selection score of each cell and a 4096-bin histogram of the
// top 12 bits of its ordered key, which it adds into the head's histogram.
// The last workgroup of a head to finish (an atomic counter, no waiting)
// then selects that head's top-K cells:
//   * the composite key of a cell is (ordered fp32 score, then the inverse
//     flat index), so all keys differ and "the first K cells in (score
//     descending, flat index ascending)" are exactly the K largest keys;
//   * a radix select walks the key from the top: the global histogram fixes
//     the first 12 bits, further 12-bit passes over the head run only while
//     the current bin holds more than kCap cells, then the remaining cells are
//     copied into LDS and 8-bit passes there find the K-th largest key T;
//   * the selected set {key >= T} is written as a bitmap, as CSR (row_ptr,
//     col ascending) and as the attention work list (block row, chunk of at
//     most kChunk selected key blocks).
// The translation unit is built with -ffp-contract=off so that every fp32
// operation is the one written.
#include "mra_common.h"

namespace mra {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRT = 16;     // block rows per workgroup
constexpr int kCT = 128;    // key blocks per logits tile
constexpr int kCap = 4096;  // selection candidates held in LDS

// ---------------------------------------------------------------- LDS plan
// logits phase:  qT[64][kRT] | kT[64][kCT] | srow[kRT][nb] | cntv[nb] | hist[4096] | small
// select phase:  hist[4096] | cand[kCap] (u64) | bitmap[nb][words] | rm[nb] | cntv[nb]
//                | rc[nb+1] | ic[nb+1] | scan[64] | small
struct LogitsLds {
    size_t qT, kT, srow, cntv, hist, small, total;
};
struct SelectLds {
    size_t hist, cand, bitmap, rm, cntv, rc, ic, scan, small, total;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

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

__host__ __device__ inline SelectLds select_lds(int nb) {
    SelectLds L;
    const int words = (nb + 31) / 32;
    size_t o = 0;
    L.hist = o; o = align16(o + kHistBins * 4);
    L.cand = o; o = align16(o + (size_t)kCap * 8);
    L.bitmap = o; o = align16(o + (size_t)nb * words * 4);
    L.rm = o; o = align16(o + (size_t)nb * 4);
    L.cntv = o; o = align16(o + (size_t)nb * 4);
    L.rc = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.ic = o; o = align16(o + (size_t)(nb + 1) * 4);
    L.scan = o; o = align16(o + 64 * 4);
    L.small = o; o = align16(o + 64 * 8);
    L.total = o;
    return L;
}

// Exclusive scan of one int per thread over the workgroup (kThreads).
// Returns the exclusive prefix; *total gets the sum.  Uses scan[kWaves].
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
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < kWaves; w++) {
            int t = scan[w];
            scan[w] = run;
            run += t;
        }
        scan[kWaves] = run;
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
    const int t = threadIdx.x;
    const int rt = kThreads - 1 - t;   // reversed: thread rt scans the top bins first
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

__device__ __forceinline__ uint64_t key_of(const float* __restrict__ S, const float* rm,
                                          const int* cntv, int nb, int i, int j, int pf, int pd) {
    const float s = cell_score(S[(size_t)i * nb + j], rm[i], i, j, cntv[i] > 0, cntv[j] > 0, pf, pd);
    return cell_key64(float_key(s), (uint32_t)(i * nb + j));
}

// kGiven: the logits are already in p.logits (selector hook); skip step 1.
template <bool kGiven>
__global__ __launch_bounds__(kThreads) void logits_select_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = p.nb;
    const int tiles_per_head = (nb + kRT - 1) / kRT;
    const int bh = blockIdx.x / tiles_per_head;
    const int row0 = (blockIdx.x - bh * tiles_per_head) * kRT;
    const int b = bh / p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float tau = (float)(1.0 / __builtin_sqrt((double)p.d));

    // ------------------------------------------------------------ logits
    {
        const LogitsLds L = logits_lds(nb);
        float* qT = reinterpret_cast<float*>(smem + L.qT);
        float* kT = reinterpret_cast<float*>(smem + L.kT);
        float* srow = reinterpret_cast<float*>(smem + L.srow);
        int* cntv = reinterpret_cast<int*>(smem + L.cntv);
        uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist);
        float* rmax = reinterpret_cast<float*>(smem + L.small);

        for (int j = tid; j < nb; j += kThreads) cntv[j] = p.cnt[b * nb + j];
        for (int x = tid; x < kHistBins; x += kThreads) hist[x] = 0u;
        const float* qh = p.qhat + (size_t)bh * nb * kHeadDim;
        const float* kh = p.khat + (size_t)bh * nb * kHeadDim;
        // qT[c][r] = qhat[row0 + r][c]
        for (int x = tid; x < (kGiven ? 0 : kRT * kHeadDim); x += kThreads) {
            const int r = x / kHeadDim, c = x - r * kHeadDim;
            qT[c * kRT + r] = (row0 + r < nb) ? qh[(size_t)(row0 + r) * kHeadDim + c] : 0.0f;
        }
        const int r0 = 2 * wave;          // this wave's two block rows
        if (kGiven) {
            for (int x = tid; x < kRT * nb; x += kThreads) {
                const int r = x / nb, j = x - r * nb;
                srow[x] = (row0 + r < nb) ? p.logits[((size_t)bh * nb + row0 + r) * nb + j] : 0.0f;
            }
        }
        for (int j0 = 0; j0 < (kGiven ? 0 : nb); j0 += kCT) {
            __syncthreads();
            // kT[c][jj] = khat[j0 + jj][c]
            for (int x = tid; x < kCT * (kHeadDim / 4); x += kThreads) {
                const int jj = x % kCT, c4 = (x / kCT) * 4;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (j0 + jj < nb) v = *reinterpret_cast<const float4*>(kh + (size_t)(j0 + jj) * kHeadDim + c4);
                kT[(c4 + 0) * kCT + jj] = v.x;
                kT[(c4 + 1) * kCT + jj] = v.y;
                kT[(c4 + 2) * kCT + jj] = v.z;
                kT[(c4 + 3) * kCT + jj] = v.w;
            }
            __syncthreads();
            float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
#pragma unroll 8
            for (int c = 0; c < kHeadDim; c++) {
                const float2 qv = *reinterpret_cast<const float2*>(qT + c * kRT + r0);
                const float2 kv = *reinterpret_cast<const float2*>(kT + c * kCT + 2 * lane);
                a00 = __builtin_fmaf(qv.x, kv.x, a00);
                a01 = __builtin_fmaf(qv.x, kv.y, a01);
                a10 = __builtin_fmaf(qv.y, kv.x, a10);
                a11 = __builtin_fmaf(qv.y, kv.y, a11);
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
            const float s = cell_score(sv, rmax[r], i, j, cntv[i] > 0, cntv[j] > 0, p.prior_first,
                                       p.prior_diag);
            atomicAdd(&hist[float_key(s) >> (32 - kHistBits)], 1u);
        }
        for (int r = tid; r < kRT; r += kThreads)
            if (row0 + r < nb) p.rowmax[(size_t)bh * nb + row0 + r] = rmax[r];
        __syncthreads();
        uint32_t* gh = p.hist + (size_t)bh * kHistBins;
        for (int x = tid; x < kHistBins; x += kThreads)
            if (hist[x]) atomicAdd(&gh[x], hist[x]);
        // publish, then count this workgroup as done for the head
        __threadfence();
        __syncthreads();
        uint32_t* flag = reinterpret_cast<uint32_t*>(smem + L.small) + 32;
        if (tid == 0) flag[0] = atomicAdd(&p.done[bh], 1u) == (uint32_t)(tiles_per_head - 1) ? 1u : 0u;
        __syncthreads();
        const bool last = flag[0] != 0;
        __syncthreads();
        if (!last) return;
        __threadfence();
    }

    // ------------------------------------------------------------ select
    const SelectLds L = select_lds(nb);
    const int words = p.words;
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist);
    uint64_t* cand = reinterpret_cast<uint64_t*>(smem + L.cand);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + L.bitmap);
    float* rm = reinterpret_cast<float*>(smem + L.rm);
    int* cntv = reinterpret_cast<int*>(smem + L.cntv);
    int* rc = reinterpret_cast<int*>(smem + L.rc);
    int* ic = reinterpret_cast<int*>(smem + L.ic);
    int* scan = reinterpret_cast<int*>(smem + L.scan);
    uint32_t* small = reinterpret_cast<uint32_t*>(smem + L.small);
    const float* S = p.logits + (size_t)bh * nb * nb;
    const int ncell = nb * nb;
    const int pf = p.prior_first, pd = p.prior_diag;

    for (int j = tid; j < nb; j += kThreads) {
        cntv[j] = p.cnt[b * nb + j];
        rm[j] = p.rowmax[(size_t)bh * nb + j];
    }
    for (int x = tid; x < kHistBins; x += kThreads) hist[x] = p.hist[(size_t)bh * kHistBins + x];
    __syncthreads();

    uint32_t need = (uint32_t)p.K;
    BinPick bp = pick_bin(hist, need, scan, small);
    need -= bp.above;
    uint64_t prefix = bp.bin;
    int pbits = kHistBits;
    uint32_t count = bp.count;

    // further 12-bit passes over the head while the bin is too large for LDS
    while (count > (uint32_t)kCap && pbits < 64) {
        const int db = (64 - pbits) < 12 ? (64 - pbits) : 12;
        for (int x = tid; x < kHistBins; x += kThreads) hist[x] = 0u;
        __syncthreads();
        for (int f = tid; f < ncell; f += kThreads) {
            const int i = f / nb, j = f - i * nb;
            const uint64_t k64 = key_of(S, rm, cntv, nb, i, j, pf, pd);
            if ((k64 >> (64 - pbits)) == prefix)
                atomicAdd(&hist[(uint32_t)((k64 >> (64 - pbits - db)) & ((1ull << db) - 1))], 1u);
        }
        __syncthreads();
        bp = pick_bin(hist, need, scan, small);
        need -= bp.above;
        prefix = (prefix << db) | bp.bin;
        pbits += db;
        count = bp.count;
    }

    // copy the cells of the bin into LDS
    if (tid == 0) small[8] = 0u;
    __syncthreads();
    for (int f0 = 0; f0 < ncell; f0 += kThreads) {
        const int f = f0 + tid;
        bool hit = false;
        uint64_t k64 = 0;
        if (f < ncell) {
            const int i = f / nb, j = f - i * nb;
            k64 = key_of(S, rm, cntv, nb, i, j, pf, pd);
            hit = (k64 >> (64 - pbits)) == prefix;
        }
        const uint64_t m = __ballot(hit);
        if (m) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&small[8], (uint32_t)__popcll(m));
            base = __shfl(base, 0, 64);
            if (hit) {
                const uint32_t pos = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
                if (pos < (uint32_t)kCap) cand[pos] = k64;
            }
        }
    }
    __syncthreads();
    const uint32_t ncand = small[8] < (uint32_t)kCap ? small[8] : (uint32_t)kCap;
    if (tid == 0 && small[8] != count) atomicOr(reinterpret_cast<unsigned int*>(p.error), 1u);
    __syncthreads();

    // 8-bit passes in LDS until the K-th largest key is pinned down
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

    // bitmap of the selected cells ({key >= T}) and per-row counts
    for (int i = wave; i < nb; i += kWaves) {
        int rcount = 0;
        for (int j0 = 0; j0 < nb; j0 += 64) {
            const int j = j0 + lane;
            const bool sel = j < nb && key_of(S, rm, cntv, nb, i, j, pf, pd) >= T;
            const uint64_t m = __ballot(sel);
            rcount += __popcll(m);
            if (lane == 0) {
                bitmap[i * words + j0 / 32] = (uint32_t)m;
                if (j0 / 32 + 1 < words) bitmap[i * words + j0 / 32 + 1] = (uint32_t)(m >> 32);
            }
        }
        if (lane == 0) rc[i] = rcount;
    }
    __syncthreads();

    // CSR row pointers and work-item pointers (nb <= kThreads rows per pass)
    int row_base = 0, item_base = 0;
    int32_t* row_ptr = p.row_ptr + (size_t)bh * (nb + 1);
    int32_t* item_ptr = p.item_ptr + (size_t)bh * (nb + 1);
    for (int i0 = 0; i0 < nb; i0 += kThreads) {
        const int i = i0 + tid;
        const int c = i < nb ? rc[i] : 0;
        const int it = i < nb ? (c > 0 ? (c + kChunk - 1) / kChunk : 1) : 0;
        int tc, ti;
        const int ec = block_excl_scan(c, scan, &tc);
        const int ei = block_excl_scan(it, scan, &ti);
        if (i < nb) {
            row_ptr[i] = row_base + ec;
            item_ptr[i] = item_base + ei;
            rc[i] = row_base + ec;     // becomes the CSR offset
            ic[i] = item_base + ei;
        }
        row_base += tc;
        item_base += ti;
    }
    if (tid == 0) {
        row_ptr[nb] = row_base;
        item_ptr[nb] = item_base;
        p.n_items[bh] = item_base;
        if ((int64_t)row_base != p.K || item_base > p.max_items)
            atomicOr(reinterpret_cast<unsigned int*>(p.error), 2u);
    }
    __syncthreads();

    // column lists, bitmap and work items
    int2* items = p.items + (size_t)bh * p.max_items;
    int32_t* col = p.col + (size_t)bh * p.K;
    uint32_t* gbits = p.selbits + (size_t)bh * nb * words;
    for (int x = tid; x < nb * words; x += kThreads) gbits[x] = bitmap[x];
    for (int i = wave; i < nb; i += kWaves) {
        int pos = rc[i];
        for (int j0 = 0; j0 < nb; j0 += 64) {
            const int j = j0 + lane;
            bool sel = false;
            if (j < nb) sel = (bitmap[i * words + (j >> 5)] >> (j & 31)) & 1u;
            const uint64_t m = __ballot(sel);
            if (sel) {
                const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
                if (at < p.K) col[at] = j;
            }
            pos += __popcll(m);
        }
        const int first = ic[i];
        const int nsel = pos - rc[i];
        const int nit = nsel > 0 ? (nsel + kChunk - 1) / kChunk : 1;
        for (int c = lane; c < nit; c += 64)
            if (first + c < p.max_items) items[first + c] = make_int2(i, c);
    }
}

}  // namespace

size_t logits_select_lds_bytes(int nb) {
    const size_t a = logits_lds(nb).total, s = select_lds(nb).total;
    return a > s ? a : s;
}

template <bool kGiven>
static hipError_t launch_ls(const Params& p, hipStream_t s) {
    const int tiles_per_head = (p.nb + kRT - 1) / kRT;
    const size_t lds = logits_select_lds_bytes(p.nb);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&logits_select_kernel<kGiven>), hipFuncAttributeMaxDynamicSharedMemorySize,
        160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(logits_select_kernel<kGiven>, dim3(p.BH * tiles_per_head), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_logits_select(const Params& p, hipStream_t s) { return launch_ls<false>(p, s); }
hipError_t launch_select_from_logits(const Params& p, hipStream_t s) { return launch_ls<true>(p, s); }

}  // namespace mra
