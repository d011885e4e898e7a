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

__global__ __launch_bounds__(TT) void topk_rows(const float* __restrict__ scores,
                                                int32_t* __restrict__ idx, int T, int N, int k,
                                                int q_offset) {
    __shared__ uint32_t hist[BINS];
    __shared__ int32_t listA[KMAX];
    __shared__ int32_t listB[KMAX];
    __shared__ uint32_t ckey[CAP];
    __shared__ int32_t cidx[CAP];
    __shared__ uint32_t sh[NW + 1];
    __shared__ uint32_t res[3];

    const int tid = threadIdx.x;
    const int t = blockIdx.x, b = blockIdx.y;
    const size_t row = (size_t)b * T + t;
    const int n_cand = (int)min((long long)N, (long long)q_offset + t + 1);
    int32_t* __restrict__ out = idx + row * k;

    if (n_cand <= k) {  // every candidate is kept
        for (int i = tid; i < k; i += TT) out[i] = i < n_cand ? i : -1;
        return;
    }
    const uint32_t n = (uint32_t)k;
    const float* __restrict__ s = scores + row * N;
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

}  // namespace

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

dsa_status launch_topk(const float* scores, int32_t* idx, int B, int T, int N, int k,
                       int q_offset, void*, hipStream_t stream) {
    if (k > KMAX) return DSA_ERR_UNSUPPORTED;
    if (B > 65535) return DSA_ERR_UNSUPPORTED;
    topk_rows<<<dim3(T, B), TT, 0, stream>>>(scores, idx, T, N, k, q_offset);
    return launch_status();
}

}  // namespace dsa
