// Device code shared by the top-k selection kernels (included by the
// translation units that select; everything is internal to each of them).
//
// Keys: an order-preserving uint32 image of the fp32 score (fkey);
// selection is a radix select over a 12-bit first digit (4096 bins) and two
// 10-bit digits, ties broken by the lower token index.
#pragma once

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int TT = 1024;         // threads per row
constexpr int NW = TT / 64;      // waves per row
constexpr int BINS = seg::kBins; // first digit: key bits 31..20
constexpr int CAP = 4096;        // LDS candidate capacity (two workgroups per CU)
constexpr int KMAX = seg::kMaxK;

// Inclusive sum over the 64 lanes of a wave: DPP row_shr 1, 2, 4, 8 within
// rows of 16 lanes, then row_bcast 15 and 31 across rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const int lane = threadIdx.x & 63, rl = lane & 15;
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x111, 0xf, 0xf, false);
    if (rl >= 1) v += t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x112, 0xf, 0xf, false);
    if (rl >= 2) v += t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xf, 0xf, false);
    if (rl >= 4) v += t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x118, 0xf, 0xf, false);
    if (rl >= 8) v += t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x142, 0xf, 0xf, false);
    if ((lane & 31) >= 16) v += t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x143, 0xf, 0xf, false);
    if (lane >= 32) v += t;
    return v;
}

// Exclusive prefix sum of v over the workgroup of NTH threads (thread
// order); *total gets the sum.  sh holds NTH/64 + 1 words.  Contains
// barriers: every thread must call it.
template <int NTH = TT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    constexpr int NWV = NTH / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t x = lane < NWV ? sh[lane] : 0u;
        const uint32_t xi = wave_incl_scan(x);
        if (lane < NWV) sh[lane] = xi - x;
        if (lane == NWV - 1) sh[NWV] = xi;
    }
    __syncthreads();
    const uint32_t r = sh[wave] + incl - v;
    *total = sh[NWV];
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
// to res.  Every thread of the NTH-thread workgroup must call it.
template <int NTH = TT>
__device__ void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* sh, uint32_t* res) {
    const int per = (nb + NTH - 1) / NTH;    // bins per thread
    const int hi = nb - per * (int)threadIdx.x;  // this thread owns bins [hi-per, hi)
    uint32_t cnt = 0;
    for (int i = 1; i <= per; ++i)
        if (hi - i >= 0) cnt += hist[hi - i];
    uint32_t total;
    const uint32_t above = block_excl_scan<NTH>(cnt, sh, &total);
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

// ---------------------------------------------------------------------------
// Tail shared by the selections that finish from an LDS candidate list.

// Among the candidates with key == kthr (n_tie of them), keep the r lowest
// indices: returns inv_thr such that exactly those ties have ~index >= inv_thr
// (0 when every tie is kept).  Radix select on ~index (larger = lower index)
// with digits of 12, 10 and 10 bits.  hist needs BINS words.  Every thread of
// the NTH-thread workgroup must call it.
template <int NTH = TT>
__device__ uint32_t tie_threshold(const uint32_t* ckey, const int32_t* cidx, int n_c, uint32_t kthr,
                                  uint32_t n_tie, uint32_t r, uint32_t* hist, uint32_t* sh,
                                  uint32_t* res) {
    if (n_tie <= r) return 0u;
    uint32_t prefix = 0u, need = r;
    int shift = 32;
    while (shift > 0) {
        const int d = shift == 32 ? 12 : 10;
        const uint32_t nb = 1u << d;
        for (int i = threadIdx.x; i < (int)nb; i += NTH) hist[i] = 0u;
        __syncthreads();
        #pragma unroll 1
        for (int i = threadIdx.x; i < n_c; i += NTH) {
            const uint32_t inv = ~(uint32_t)cidx[i];
            const bool pre = shift == 32 || (inv >> shift) == prefix;
            if (ckey[i] == kthr && pre) atomicAdd(&hist[(inv >> (shift - d)) & (nb - 1u)], 1u);
        }
        __syncthreads();
        find_bin<NTH>(hist, (int)nb, need, sh, res);
        need -= res[1];
        prefix = (prefix << d) | res[0];
        shift -= d;
    }
    return prefix;
}

constexpr int BM_BITS = BINS * 32;  // index window of one bitmap pass

// Write the picks in ascending index order: the n_sure indices of `sure`
// (global memory) and the candidates with key > kthr, or key == kthr and
// ~index >= inv_thr, all below n_cand.  A bitmap over BM_BITS indices at a
// time (bm: BINS words) and a block scan of the per-thread popcounts give
// every pick its output slot.  Every thread of the NTH-thread workgroup must
// call it.
template <int NTH = TT>
__device__ void emit_ascending(const int32_t* __restrict__ sure, int n_sure, const uint32_t* ckey,
                               const int32_t* cidx, int n_c, uint32_t kthr, uint32_t inv_thr,
                               int n_cand, int32_t* __restrict__ out, uint32_t* bm, uint32_t* sh) {
    const int tid = threadIdx.x;
    uint32_t emitted = 0;
    for (int w0 = 0; w0 < n_cand; w0 += BM_BITS) {
        for (int i = tid; i < BINS; i += NTH) bm[i] = 0u;
        __syncthreads();
        #pragma unroll 1
        for (int i = tid; i < n_sure; i += NTH) {
            const int e = sure[i] - w0;
            if (e >= 0 && e < BM_BITS) atomicOr(&bm[e >> 5], 1u << (e & 31));
        }
        #pragma unroll 1
        for (int i = tid; i < n_c; i += NTH) {
            const uint32_t key = ckey[i];
            const bool take = key > kthr || (key == kthr && ~(uint32_t)cidx[i] >= inv_thr);
            const int e = cidx[i] - w0;
            if (take && e >= 0 && e < BM_BITS) atomicOr(&bm[e >> 5], 1u << (e & 31));
        }
        __syncthreads();
        constexpr int WPT = BINS / NTH;  // bitmap words per thread
        uint32_t m[WPT], cnt = 0;
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            m[j] = bm[WPT * tid + j];
            cnt += __popc(m[j]);
        }
        uint32_t total;
        uint32_t p = emitted + block_excl_scan<NTH>(cnt, sh, &total);
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

// Exact top-k among n_c >= k candidates (keys ckey, token indices cidx, any
// order) written to out in ascending index order: the k-th key by three radix
// digits (12, 10, 10 bits), the lowest-index ties, bitmap emission over
// [0, n_cand).  hist: BINS words of LDS; sh: NTH/64 + 1 words; res: 3.
// PADDED: the list also holds unused slots of key 0 below every candidate
// (the one-pass row selection); they are left out of the first histogram,
// where they would all hit one bin, and change no count above that bin.
template <int NTH = TT, bool PADDED = false>
__device__ __forceinline__ void select_candidates(const uint32_t* ckey, const int32_t* cidx, int n_c, int k,
                                  int n_cand, int32_t* __restrict__ out, uint32_t* hist,
                                  uint32_t* sh, uint32_t* res) {
    const int tid = threadIdx.x;
    for (int i = tid; i < BINS; i += NTH) hist[i] = 0u;
    __syncthreads();
    #pragma unroll 1
    for (int i = tid; i < n_c; i += NTH)
        if (!PADDED || ckey[i] != 0u) atomicAdd(&hist[ckey[i] >> 20], 1u);
    __syncthreads();
    find_bin<NTH>(hist, BINS, (uint32_t)k, sh, res);
    const uint32_t b1 = res[0], r1 = (uint32_t)k - res[1];
    for (int i = tid; i < 1024; i += NTH) hist[i] = 0u;
    __syncthreads();
    #pragma unroll 1
    for (int i = tid; i < n_c; i += NTH)
        if ((ckey[i] >> 20) == b1) atomicAdd(&hist[(ckey[i] >> 10) & 1023u], 1u);
    __syncthreads();
    find_bin<NTH>(hist, 1024, r1, sh, res);
    const uint32_t p2 = (b1 << 10) | res[0], r2 = r1 - res[1];
    for (int i = tid; i < 1024; i += NTH) hist[i] = 0u;
    __syncthreads();
    #pragma unroll 1
    for (int i = tid; i < n_c; i += NTH)
        if ((ckey[i] >> 10) == p2) atomicAdd(&hist[ckey[i] & 1023u], 1u);
    __syncthreads();
    find_bin<NTH>(hist, 1024, r2, sh, res);
    const uint32_t kthr = (p2 << 10) | res[0], n_tie = res[2], r3 = r2 - res[1];
    const uint32_t inv_thr = tie_threshold<NTH>(ckey, cidx, n_c, kthr, n_tie, r3, hist, sh, res);
    emit_ascending<NTH>(nullptr, 0, ckey, cidx, n_c, kthr, inv_thr, n_cand, out, hist, sh);
}

// Candidate threshold from a sample of a row's keys: the key of the r-th
// largest of the S sample keys in skey, rounded down to its top 22 bits, with
// r = mu + c1 sqrt(mu) + c0 and mu = S k / n_cand (the expected number of
// samples among the row's top k); 0 (every key passes) when r >= S.  Keys at
// or above it hold the row's top k unless the sample is far from typical.
// hist: BINS words; every thread of the NTH-thread workgroup must call it.
template <int NTH = TT>
__device__ uint32_t sample_threshold(const uint32_t* skey, int S, int k, int n_cand, float c1,
                                     float c0, uint32_t* hist, uint32_t* sh, uint32_t* res) {
    const float mu = (float)S * (float)k / (float)n_cand;
    const int r = (int)ceilf(mu + c1 * sqrtf(mu) + c0);
    if (r >= S) return 0u;
    const int tid = threadIdx.x;
    for (int i = tid; i < BINS; i += NTH) hist[i] = 0u;
    __syncthreads();
    #pragma unroll 1
    for (int i = tid; i < S; i += NTH) atomicAdd(&hist[skey[i] >> 20], 1u);
    __syncthreads();
    find_bin<NTH>(hist, BINS, (uint32_t)r, sh, res);
    const uint32_t b1 = res[0], r2 = (uint32_t)r - res[1];
    for (int i = tid; i < 1024; i += NTH) hist[i] = 0u;
    __syncthreads();
    #pragma unroll 1
    for (int i = tid; i < S; i += NTH)
        if ((skey[i] >> 20) == b1) atomicAdd(&hist[(skey[i] >> 10) & 1023u], 1u);
    __syncthreads();
    find_bin<NTH>(hist, 1024, r2, sh, res);
    return (b1 << 20) | (res[0] << 10);
}

}  // namespace
}  // namespace dsa
