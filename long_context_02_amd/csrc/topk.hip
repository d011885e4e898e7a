// Per-query causal top-k token selection on gfx950.
//
// Selection ("Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture: DSA
// (§2.1)"): query t keeps the k tokens with the largest index scores among
// its causal candidates s < min(N, q_offset + t + 1).  Ties go to the lower
// index, -0 equals +0, NaN ranks lowest; the kept indices are written in
// ascending order and padded with -1.
//
// One 1024-thread workgroup per row, radix select on an order-preserving
// 32-bit key:
//   pass 1 (HBM)  LDS histogram of the top 12 key bits -> the bin b1 holding
//                 the k-th largest key, the count above it and in it;
//   pass 2 (HBM)  ordered compaction: keys above b1 go to list A (they are
//                 kept for sure), keys inside b1 go to an LDS candidate list
//                 C with their indices, both in index order (a block-wide
//                 exclusive scan over per-thread counts built from
//                 wave-level prefix sums);
//   in LDS        two more 10-bit digits over C give the exact k-th key K*
//                 and how many of the keys equal to K* to keep; an ordered
//                 scan over C keeps every key > K* and the lowest-index keys
//                 == K* (list B);
//   merge         A and B are both ascending; each element's output slot is
//                 its rank in its own list plus its rank in the other.
// When bin b1 holds more keys than the LDS list can take (e.g. a row of
// identical scores) the remaining digits are resolved with further HBM
// passes and a final ordered emission pass over the row.
//
// Batches of few rows (decode: one row per sequence) instead split every row
// over several workgroups; see the segmented path below.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int TT = 1024;         // threads per row
constexpr int NW = TT / 64;      // waves per row
constexpr int BINS = 4096;       // first digit: key bits 31..20
constexpr int CAP = 6144;        // LDS candidate capacity
constexpr int KMAX = 2048;

// Order-preserving map float -> uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0u) return 0x80000000u;                        // -0 == +0
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0u;   // NaN lowest
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t n = __shfl_up(v, o, 64);
        if (lane >= o) v += n;
    }
    return v;
}

// Exclusive prefix sum of v over the workgroup (thread order); *total gets
// the sum.  Contains barriers: every thread must call it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t x = lane < NW ? sh[lane] : 0u;
        const uint32_t xi = wave_incl_scan(x);
        if (lane < NW) sh[lane] = xi - x;
        if (lane == NW - 1) sh[NW] = xi;
    }
    __syncthreads();
    const uint32_t r = sh[wave] + incl - v;
    *total = sh[NW];
    __syncthreads();
    return r;
}

// Four consecutive scores starting at e (vector load when aligned and whole).
__device__ __forceinline__ void load4(const float* __restrict__ s, int e, int n, bool vec, float* v) {
    if (vec && e + 3 < n) {
        const float4 x = *reinterpret_cast<const float4*>(s + e);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = e + j < n ? s[e + j] : 0.f;
    }
}

// Find, over nb histogram bins read in descending bin order, the bin that
// holds the need-th largest element.  Writes (bin, count above, count in bin)
// to res.  Every thread must call it; nb <= 4*TT.
__device__ void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* sh, uint32_t* res) {
    const int per = (nb + TT - 1) / TT;      // bins per thread (1 or 4)
    const int hi = nb - per * (int)threadIdx.x;  // this thread owns bins [hi-per, hi)
    uint32_t cnt = 0;
    for (int i = 1; i <= per; ++i)
        if (hi - i >= 0) cnt += hist[hi - i];
    uint32_t total;
    const uint32_t above = block_excl_scan(cnt, sh, &total);
    if (cnt > 0 && above < need && above + cnt >= need) {
        uint32_t acc = above;
        for (int i = 1; i <= per; ++i) {
            const uint32_t h = hist[hi - i];
            if (acc + h >= need) {
                res[0] = (uint32_t)(hi - i);
                res[1] = acc;
                res[2] = h;
                break;
            }
            acc += h;
        }
    }
    __syncthreads();
}

__device__ __forceinline__ int lower_bound(const int32_t* a, int n, int32_t v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// LDS of the single-workgroup row selection, carved from one buffer so the
// segmented path can reuse it as its fallback.
struct RowLds {
    uint32_t* hist;   // BINS
    int32_t* listA;   // KMAX
    int32_t* listB;   // KMAX
    uint32_t* ckey;   // CAP
    int32_t* cidx;    // CAP
    uint32_t* sh;     // NW + 1
    uint32_t* res;    // 3
};
constexpr int ROW_LDS_WORDS = BINS + 2 * KMAX + 2 * CAP + NW + 1 + 3;

__device__ RowLds carve_row_lds(uint32_t* base) {
    RowLds L;
    L.hist = base;
    L.listA = reinterpret_cast<int32_t*>(L.hist + BINS);
    L.listB = L.listA + KMAX;
    L.ckey = reinterpret_cast<uint32_t*>(L.listB + KMAX);
    L.cidx = reinterpret_cast<int32_t*>(L.ckey + CAP);
    L.sh = reinterpret_cast<uint32_t*>(L.cidx + CAP);
    L.res = L.sh + NW + 1;
    return L;
}

// Top-k of one row by one 1024-thread workgroup (n_cand > k).
__device__ void select_row(const float* __restrict__ s, int32_t* __restrict__ out, int n_cand, int k,
                           const RowLds& L) {
    uint32_t* hist = L.hist;
    int32_t* listA = L.listA;
    int32_t* listB = L.listB;
    uint32_t* ckey = L.ckey;
    int32_t* cidx = L.cidx;
    uint32_t* sh = L.sh;
    uint32_t* res = L.res;
    const int tid = threadIdx.x;
    const uint32_t n = (uint32_t)k;
    const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15u) == 0);

    // ---- pass 1: histogram of the top 12 key bits
    for (int i = tid; i < BINS; i += TT) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < n_cand; base += 4 * TT) {
        const int e = base + 4 * tid;
        float v[4];
        load4(s, e, n_cand, vec, v);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e + j < n_cand) atomicAdd(&hist[fkey(v[j]) >> 20], 1u);
    }
    __syncthreads();
    find_bin(hist, BINS, n, sh, res);
    const uint32_t b1 = res[0], gt1 = res[1], eq1 = res[2];

    if (eq1 <= (uint32_t)CAP) {
        // ---- pass 2: ordered compaction into list A (above b1) and C (in b1)
        uint32_t run_a = 0, run_c = 0;
        for (int base = 0; base < n_cand; base += 4 * TT) {
            const int e = base + 4 * tid;
            float v[4];
            load4(s, e, n_cand, vec, v);
            uint32_t key[4], na = 0, nc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                key[j] = fkey(v[j]);
                const bool ok = e + j < n_cand;
                na += (ok && (key[j] >> 20) > b1);
                nc += (ok && (key[j] >> 20) == b1);
            }
            uint32_t tot;
            const uint32_t ex = block_excl_scan(na | (nc << 16), sh, &tot);
            uint32_t pa = run_a + (ex & 0xffffu), pc = run_c + (ex >> 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (e + j >= n_cand) continue;
                const uint32_t d = key[j] >> 20;
                if (d > b1) {
                    listA[pa++] = e + j;
                } else if (d == b1) {
                    ckey[pc] = key[j];
                    cidx[pc] = e + j;
                    ++pc;
                }
            }
            run_a += tot & 0xffffu;
            run_c += tot >> 16;
        }
        __syncthreads();

        // ---- digits 2 and 3 inside C
        const int nc = (int)eq1;
        const uint32_t r1 = n - gt1;
        for (int i = tid; i < 1024; i += TT) hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < nc; i += TT) atomicAdd(&hist[(ckey[i] >> 10) & 1023u], 1u);
        __syncthreads();
        find_bin(hist, 1024, r1, sh, res);
        const uint32_t b2 = res[0], gt2 = res[1];
        const uint32_t r2 = r1 - gt2;
        for (int i = tid; i < 1024; i += TT) hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < nc; i += TT)
            if (((ckey[i] >> 10) & 1023u) == b2) atomicAdd(&hist[ckey[i] & 1023u], 1u);
        __syncthreads();
        find_bin(hist, 1024, r2, sh, res);
        const uint32_t b3 = res[0], gt3 = res[1];
        const uint32_t kstar = (b1 << 20) | (b2 << 10) | b3;
        const uint32_t r3 = r2 - gt3;  // keys == K* to keep, lowest indices first

        // ---- ordered selection from C into list B
        uint32_t run_g = 0, run_t = 0;
        for (int base = 0; base < nc; base += TT) {
            const int i = base + tid;
            const bool ok = i < nc;
            const uint32_t key = ok ? ckey[i] : 0u;
            const uint32_t g = ok && key > kstar, tie = ok && key == kstar;
            uint32_t tot;
            const uint32_t ex = block_excl_scan(g | (tie << 16), sh, &tot);
            const uint32_t tie_before = run_t + (ex >> 16);
            const uint32_t pos = run_g + (ex & 0xffffu) + min(tie_before, r3);
            if (g || (tie && tie_before < r3)) listB[pos] = cidx[i];
            run_g += tot & 0xffffu;
            run_t += tot >> 16;
        }
        __syncthreads();

        // ---- merge the two ascending lists
        const int na = (int)gt1, nb = (int)r1;
        for (int i = tid; i < na; i += TT) {
            const int32_t v = listA[i];
            out[i + lower_bound(listB, nb, v)] = v;
        }
        for (int j = tid; j < nb; j += TT) {
            const int32_t v = listB[j];
            out[j + lower_bound(listA, na, v)] = v;
        }
        return;
    }

    // ---- fallback: resolve the remaining digits over HBM, then emit in order
    uint32_t prefix = b1, need = n - gt1;
    int shift = 20;
    while (shift > 0) {
        const int d = shift >= 10 ? 10 : shift;
        const uint32_t nbin = 1u << d;
        for (int i = tid; i < (int)nbin; i += TT) hist[i] = 0u;
        __syncthreads();
        for (int base = 0; base < n_cand; base += 4 * TT) {
            const int e = base + 4 * tid;
            float v[4];
            load4(s, e, n_cand, vec, v);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = fkey(v[j]);
                if (e + j < n_cand && (key >> shift) == prefix)
                    atomicAdd(&hist[(key >> (shift - d)) & (nbin - 1u)], 1u);
            }
        }
        __syncthreads();
        find_bin(hist, (int)nbin, need, sh, res);
        need -= res[1];
        prefix = (prefix << d) | res[0];
        shift -= d;
    }
    const uint32_t kstar = prefix, r = need;
    uint32_t run_g = 0, run_t = 0;
    for (int base = 0; base < n_cand; base += 4 * TT) {
        const int e = base + 4 * tid;
        float v[4];
        load4(s, e, n_cand, vec, v);
        uint32_t key[4], ng = 0, nt = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            key[j] = fkey(v[j]);
            const bool ok = e + j < n_cand;
            ng += ok && key[j] > kstar;
            nt += ok && key[j] == kstar;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(ng | (nt << 16), sh, &tot);
        uint32_t gb = run_g + (ex & 0xffffu), tb = run_t + (ex >> 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (e + j >= n_cand) continue;
            if (key[j] > kstar) {
                out[gb + min(tb, r)] = e + j;
                ++gb;
            } else if (key[j] == kstar) {
                if (tb < r) out[gb + tb] = e + j;
                ++tb;
            }
        }
        run_g += tot & 0xffffu;
        run_t += tot >> 16;
    }
}


__global__ __launch_bounds__(TT) void topk_rows(const float* __restrict__ scores,
                                                int32_t* __restrict__ idx, int T, int N, int k,
                                                int q_offset) {
    __shared__ uint32_t lds[ROW_LDS_WORDS];
    const int t = blockIdx.x, b = blockIdx.y;
    const size_t row = (size_t)b * T + t;
    const int n_cand = (int)min((long long)N, (long long)q_offset + t + 1);
    int32_t* __restrict__ out = idx + row * k;
    if (n_cand <= k) {  // every candidate is kept
        for (int i = threadIdx.x; i < k; i += TT) out[i] = i < n_cand ? i : -1;
        return;
    }
    select_row(scores + row * N, out, n_cand, k, carve_row_lds(lds));
}

// ---------------------------------------------------------------------------
// Segmented selection for batches of few long rows (decode): every row is
// split into SEG-element segments handled by separate workgroups.
//   topk_seg_zero      clear each row's histogram and counters
//   topk_seg_hist      LDS histogram of the top 12 key bits of a segment,
//                      added into the row's histogram in the workspace
//   topk_seg_collect   from the row histogram: the bin b1 of the k-th largest
//                      key; keys above b1 are appended to the row's list of
//                      sure picks, keys in b1 (with their index) to its
//                      candidate list (one atomic per list and workgroup)
//   topk_seg_finalize  per row: the exact k-th key among the candidates, the
//                      lowest-index ties, and the k picks written in ascending
//                      order through an index bitmap; a row whose b1 holds
//                      more than CAPG keys is selected by the single-workgroup
//                      path instead
constexpr int SEG = 16384;              // elements per segment
constexpr int STT = TT;                 // threads of the segment kernels
constexpr int CAPG = 12288;             // candidate capacity per row
constexpr int SEG_MAX_ROWS = 255;       // batches with more rows use topk_rows
// per-row workspace, in 32-bit words
constexpr int WS_HIST = 0, WS_CTR = BINS, WS_DEF = BINS + 4, WS_CKEY = WS_DEF + KMAX,
              WS_CIDX = WS_CKEY + CAPG, WS_ROW = (WS_CIDX + CAPG + 63) / 64 * 64;
// counters: [0] sure picks, [1] candidates, [2] candidate overflow flag

__device__ __forceinline__ int row_candidates(int t, int N, int q_offset) {
    return (int)min((long long)N, (long long)q_offset + t + 1);
}

__global__ __launch_bounds__(STT) void topk_seg_zero(uint32_t* __restrict__ ws) {
    uint32_t* w = ws + (size_t)blockIdx.x * WS_ROW;
    for (int i = threadIdx.x; i < WS_DEF; i += STT) w[i] = 0u;
}

__global__ __launch_bounds__(STT) void topk_seg_hist(const float* __restrict__ scores,
                                                     uint32_t* __restrict__ ws, int T, int N, int k,
                                                     int q_offset) {
    __shared__ uint32_t hist[BINS];
    const int row = blockIdx.y, t = row % T;
    const int n_cand = row_candidates(t, N, q_offset);
    const int s0 = blockIdx.x * SEG, s1 = min(n_cand, s0 + SEG);
    if (n_cand <= k || s0 >= s1) return;
    const float* __restrict__ s = scores + (size_t)row * N;
    const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15u) == 0);
    for (int i = threadIdx.x; i < BINS; i += STT) hist[i] = 0u;
    __syncthreads();
    constexpr int PER = SEG / (4 * STT);  // 4-key groups per thread
    float v[PER][4];
#pragma unroll
    for (int i = 0; i < PER; ++i) load4(s, s0 + 4 * (int)threadIdx.x + 4 * STT * i, s1, vec, v[i]);
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (s0 + 4 * (int)threadIdx.x + 4 * STT * i + j < s1) atomicAdd(&hist[fkey(v[i][j]) >> 20], 1u);
    __syncthreads();
    uint32_t* gh = ws + (size_t)row * WS_ROW + WS_HIST;
    for (int i = threadIdx.x; i < BINS; i += STT)
        if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

__global__ __launch_bounds__(STT) void topk_seg_collect(const float* __restrict__ scores,
                                                        uint32_t* __restrict__ ws, int T, int N, int k,
                                                        int q_offset) {
    constexpr int PER = SEG / (4 * STT);  // 4-key groups per thread
    __shared__ uint4 kst[SEG / 4];        // the segment's keys; each thread reads back only its own
    __shared__ uint32_t hist[BINS];
    __shared__ uint32_t sh[NW + 1];
    __shared__ uint32_t res[3];
    __shared__ uint32_t base[2];
    const int row = blockIdx.y, t = row % T;
    const int n_cand = row_candidates(t, N, q_offset);
    const int s0 = blockIdx.x * SEG, s1 = min(n_cand, s0 + SEG);
    if (n_cand <= k || s0 >= s1) return;
    uint32_t* w = ws + (size_t)row * WS_ROW;
    const float* __restrict__ s = scores + (size_t)row * N;
    const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15u) == 0);
    const int tid = threadIdx.x;
    // out-of-range slots (last segment only) get key 0, in bin 0
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = s0 + 4 * tid + 4 * STT * i;
        float v[4];
        load4(s, e, s1, vec, v);
        kst[tid + STT * i] = make_uint4(fkey(v[0]), e + 1 < s1 ? fkey(v[1]) : 0u,
                                        e + 2 < s1 ? fkey(v[2]) : 0u, e + 3 < s1 ? fkey(v[3]) : 0u);
        if (e >= s1) kst[tid + STT * i].x = 0u;
    }
    for (int i = tid; i < BINS; i += STT) hist[i] = w[WS_HIST + i];
    __syncthreads();
    find_bin(hist, BINS, (uint32_t)k, sh, res);
    const uint32_t b1 = res[0], eq1 = res[2];
    if (eq1 > (uint32_t)CAPG) {  // the row takes the single-workgroup path
        if (blockIdx.x == 0 && tid == 0) w[WS_CTR + 2] = 1u;
        return;
    }
    // bin 0 slots past s1 are never above b1; they are skipped as candidates
    // when b1 is 0
    const int lim = (b1 == 0u) ? s1 : s0 + SEG;
    uint32_t nd = 0, nc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint4 q = kst[tid + STT * i];
        const int e = s0 + 4 * tid + 4 * STT * i;
        const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            nd += (kk[j] >> 20) > b1;
            nc += (kk[j] >> 20) == b1 && e + j < lim;
        }
    }
    // one scan of both counts (each below 2^16), one atomic per list
    uint32_t tot;
    const uint32_t pos = block_excl_scan((nd << 16) | nc, sh, &tot);
    if (tid == 0) {
        base[0] = (tot >> 16) ? atomicAdd(&w[WS_CTR + 0], tot >> 16) : 0u;
        base[1] = (tot & 0xFFFFu) ? atomicAdd(&w[WS_CTR + 1], tot & 0xFFFFu) : 0u;
    }
    __syncthreads();
    uint32_t pd = base[0] + (pos >> 16), pc = base[1] + (pos & 0xFFFFu);
    int32_t* def = reinterpret_cast<int32_t*>(w + WS_DEF);
    uint32_t* ckey = w + WS_CKEY;
    int32_t* cidx = reinterpret_cast<int32_t*>(w + WS_CIDX);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint4 q = kst[tid + STT * i];
        const int e = s0 + 4 * tid + 4 * STT * i;
        const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t bin = kk[j] >> 20;
            if (bin > b1) def[pd++] = e + j;
            else if (bin == b1 && e + j < lim) {
                ckey[pc] = kk[j];
                cidx[pc++] = e + j;
            }
        }
    }
}

constexpr int BM_BITS = BINS * 32;      // index window of one bitmap pass
constexpr int FIN_LDS_WORDS = 2 * CAPG + BINS + NW + 1 + 3;
constexpr int K3_LDS_WORDS = FIN_LDS_WORDS > ROW_LDS_WORDS ? FIN_LDS_WORDS : ROW_LDS_WORDS;

__global__ __launch_bounds__(TT) void topk_seg_finalize(const float* __restrict__ scores,
                                                        const uint32_t* __restrict__ ws,
                                                        int32_t* __restrict__ idx, int T, int N, int k,
                                                        int q_offset) {
    __shared__ uint32_t lds[K3_LDS_WORDS];
    const int row = blockIdx.x, t = row % T;
    const int tid = threadIdx.x;
    const int n_cand = row_candidates(t, N, q_offset);
    int32_t* __restrict__ out = idx + (size_t)row * k;
    if (n_cand <= k) {
        for (int i = tid; i < k; i += TT) out[i] = i < n_cand ? i : -1;
        return;
    }
    const uint32_t* w = ws + (size_t)row * WS_ROW;
    if (w[WS_CTR + 2]) {
        select_row(scores + (size_t)row * N, out, n_cand, k, carve_row_lds(lds));
        return;
    }
    uint32_t* ckey = lds;                                     // CAPG
    int32_t* cidx = reinterpret_cast<int32_t*>(ckey + CAPG);  // CAPG
    uint32_t* hist = reinterpret_cast<uint32_t*>(cidx + CAPG);  // BINS, later the bitmap
    uint32_t* sh = hist + BINS;                               // NW + 1
    uint32_t* res = sh + NW + 1;                              // 3
    const int n_def = (int)w[WS_CTR + 0], n_c = (int)w[WS_CTR + 1];
    const int32_t* gdef = reinterpret_cast<const int32_t*>(w + WS_DEF);
    for (int i = tid; i < n_c; i += TT) {
        ckey[i] = w[WS_CKEY + i];
        cidx[i] = reinterpret_cast<const int32_t*>(w + WS_CIDX)[i];
    }
    const uint32_t r1 = (uint32_t)(k - n_def);  // picks still to make among the candidates
    // digits 2 and 3 (key bits 19..10 and 9..0) give the exact k-th key
    for (int i = tid; i < 1024; i += TT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n_c; i += TT) atomicAdd(&hist[(ckey[i] >> 10) & 1023u], 1u);
    __syncthreads();
    find_bin(hist, 1024, r1, sh, res);
    const uint32_t b2 = res[0], r2 = r1 - res[1];
    for (int i = tid; i < 1024; i += TT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n_c; i += TT)
        if (((ckey[i] >> 10) & 1023u) == b2) atomicAdd(&hist[ckey[i] & 1023u], 1u);
    __syncthreads();
    find_bin(hist, 1024, r2, sh, res);
    const uint32_t b3 = res[0], n_tie = res[2];
    const uint32_t klow = (b2 << 10) | b3;  // low 20 bits of the k-th key
    const uint32_t r3 = r2 - res[1];        // ties to keep, lowest indices first
    // when not every tie is kept, the r3-th smallest tie index bounds them:
    // radix select on ~index (larger = lower index), 12 + 10 + 10 bits
    uint32_t inv_thr = 0u;  // keep ties with ~index >= inv_thr
    if (n_tie > r3) {
        uint32_t prefix = 0u, need = r3;
        int shift = 32;
        while (shift > 0) {
            const int d = shift == 32 ? 12 : 10;
            const uint32_t nb = 1u << d;
            for (int i = tid; i < (int)nb; i += TT) hist[i] = 0u;
            __syncthreads();
            for (int i = tid; i < n_c; i += TT) {
                const uint32_t inv = ~(uint32_t)cidx[i];
                const bool tie = (ckey[i] & 0xFFFFFu) == klow;
                const bool pre = shift == 32 || (inv >> shift) == prefix;
                if (tie && pre) atomicAdd(&hist[(inv >> (shift - d)) & (nb - 1u)], 1u);
            }
            __syncthreads();
            find_bin(hist, (int)nb, need, sh, res);
            need -= res[1];
            prefix = (prefix << d) | res[0];
            shift -= d;
        }
        inv_thr = prefix;
    }
    // ascending output: a bitmap over a window of BM_BITS indices at a time,
    // one bit per pick, then a scan of the per-thread popcounts
    uint32_t* bm = hist;
    uint32_t emitted = 0;
    for (int w0 = 0; w0 < n_cand; w0 += BM_BITS) {
        for (int i = tid; i < BINS; i += TT) bm[i] = 0u;
        __syncthreads();
        for (int i = tid; i < n_def; i += TT) {
            const int e = gdef[i] - w0;
            if (e >= 0 && e < BM_BITS) atomicOr(&bm[e >> 5], 1u << (e & 31));
        }
        for (int i = tid; i < n_c; i += TT) {
            const uint32_t kl = ckey[i] & 0xFFFFFu;
            const bool take = kl > klow || (kl == klow && ~(uint32_t)cidx[i] >= inv_thr);
            const int e = cidx[i] - w0;
            if (take && e >= 0 && e < BM_BITS) atomicOr(&bm[e >> 5], 1u << (e & 31));
        }
        __syncthreads();
        constexpr int WPT = BINS / TT;  // bitmap words per thread
        uint32_t m[WPT], cnt = 0;
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            m[j] = bm[WPT * tid + j];
            cnt += __popc(m[j]);
        }
        uint32_t total;
        uint32_t p = emitted + block_excl_scan(cnt, sh, &total);
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            uint32_t x = m[j];
            while (x) {
                const int b = __ffs(x) - 1;
                x &= x - 1u;
                out[p++] = w0 + 32 * (WPT * tid + j) + b;
            }
        }
        emitted += total;
    }
}

}  // namespace

size_t topk_workspace_bytes(int B, int T, int, int) {
    const long long rows = (long long)B * T;
    return rows <= SEG_MAX_ROWS ? (size_t)rows * WS_ROW * sizeof(uint32_t) : 0;
}

dsa_status launch_topk(const float* scores, int32_t* idx, int B, int T, int N, int k,
                       int q_offset, void* workspace, hipStream_t stream) {
    if (k > KMAX) return DSA_ERR_UNSUPPORTED;
    if (B > 65535) return DSA_ERR_UNSUPPORTED;
    const long long rows = (long long)B * T;
    if (rows > SEG_MAX_ROWS) {
        topk_rows<<<dim3(T, B), TT, 0, stream>>>(scores, idx, T, N, k, q_offset);
        return launch_status();
    }
    // few long rows: several workgroups per row
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    const long long n_max = std::min<long long>(N, (long long)q_offset + T);
    const int nseg = (int)((n_max + SEG - 1) / SEG);
    topk_seg_zero<<<dim3((unsigned)rows), STT, 0, stream>>>(ws);
    topk_seg_hist<<<dim3(nseg, (unsigned)rows), STT, 0, stream>>>(scores, ws, T, N, k, q_offset);
    topk_seg_collect<<<dim3(nseg, (unsigned)rows), STT, 0, stream>>>(scores, ws, T, N, k, q_offset);
    topk_seg_finalize<<<dim3((unsigned)rows), TT, 0, stream>>>(scores, ws, idx, T, N, k, q_offset);
    return launch_status();
}

}  // namespace dsa
