// FP8 index-score arithmetic shared by the kernels that compute lightning-
// indexer scores ("Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture:
// DSA (§2.1)": I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])).  A given (query,
// key) score must come out bit-identical wherever it is computed, so every
// kernel of one layout uses these helpers.
#pragma once

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int HI = 8;      // indexer heads
constexpr int DI = 128;    // indexer dim = bytes per FP8 row

// C[16x16] = A[16x128] * B[128x16], FP8 e4m3 both sides, fp32 result.
// A lane l holds row l%16, B lane l holds column l%16, each as 32 bytes of
// the 128-byte vector starting at byte 32*(l/16); A and B use the same byte
// slice, so every q byte meets the matching k byte.  C lane l holds rows
// 4*(l/16)+i (i = 0..3) of column l%16.
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 pack8(const uint4& x0, const uint4& x1) {
    return i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                 (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// ReLU as one integer max on the bit pattern: negative floats (sign bit
// set, -0 included) are negative as int32 and become +0, the rest pass
// unchanged.  (fmaxf would add a NaN-quieting max in front of every use.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// sum_j ws[j] * ReLU(D_j): acc0 holds heads 0-3, acc1 heads 4-7.
__device__ __forceinline__ float head_sum(const f32x4& acc0, const f32x4& acc1, const float* ws) {
    float s = ws[0] * relu(acc0[0]);
    s = fmaf(ws[1], relu(acc0[1]), s);
    s = fmaf(ws[2], relu(acc0[2]), s);
    s = fmaf(ws[3], relu(acc0[3]), s);
    s = fmaf(ws[4], relu(acc1[0]), s);
    s = fmaf(ws[5], relu(acc1[1]), s);
    s = fmaf(ws[6], relu(acc1[2]), s);
    s = fmaf(ws[7], relu(acc1[3]), s);
    return s;
}

// ---- tiled layout: the 16 MFMA rows are 4 queries x 4 heads ---------------
// Two MFMAs (heads 0-3, then 4-7) give lane l all 8 head dots of query
// tq0 + l/16 and key l%16; head_sum (above) in that order, then the key scale.

// Load the A fragments (one query group of 4 queries, both head halves) and
// the per-lane head weights w * q_scale of the query whose scores this lane
// produces.  Queries at or beyond T get zeros.
__device__ __forceinline__ void load_queries(const uint8_t* __restrict__ q,
                                             const float* __restrict__ qs,
                                             const float* __restrict__ w, size_t row0,
                                             int tq0, int T, int lane, i32x8* a, float* ws) {
    const int m = lane & 15, kb = lane >> 4;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int t = tq0 + (m >> 2), h = 4 * hh + (m & 3);
        if (t < T) {
            const uint4* p = reinterpret_cast<const uint4*>(q + ((row0 + t) * HI + h) * DI + 32 * kb);
            a[hh] = pack8(p[0], p[1]);
        } else {
            a[hh] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    const int t = tq0 + kb;
#pragma unroll
    for (int j = 0; j < HI; ++j)
        ws[j] = t < T ? w[(row0 + t) * HI + j] * qs[(row0 + t) * HI + j] : 0.f;
}

// ---- stream layout: the 16 MFMA rows are 2 queries x 8 heads -------------
// C lane l holds rows 4*(l/16)+i: query (l/16)/2 of the pair, heads
// 4*((l/16)&1)+i; a score's two head halves sit in lanes l and l ^ 16.

// A fragment and this lane's weights for the query pair (t_first, t_first+1);
// queries at or beyond t_lim get zeros.  *t_lane = the lane's query.
__device__ __forceinline__ void pair_operands(const uint8_t* __restrict__ q,
                                              const float* __restrict__ qs,
                                              const float* __restrict__ w, size_t row0, int t_first,
                                              int t_lim, int lane, i32x8* a, float* ws4, int* t_lane) {
    const int m = lane & 15, kb = lane >> 4;
    const int ta = t_first + (m >> 3), h = m & 7;
    if (ta < t_lim) {
        const uint4* src = reinterpret_cast<const uint4*>(q + ((row0 + ta) * HI + h) * DI + 32 * kb);
        *a = pack8(src[0], src[1]);
    } else {
        *a = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    const int tl = t_first + (kb >> 1);
    *t_lane = tl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h2 = 4 * (kb & 1) + i;
        ws4[i] = tl < t_lim ? w[(row0 + tl) * HI + h2] * qs[(row0 + tl) * HI + h2] : 0.f;
    }
}

// The lane's half of a score (its four heads), then the whole score: the two
// halves added across lanes l and l ^ 16, times the key scale.
__device__ __forceinline__ float half_score(const f32x4& acc, const float* ws4) {
    float part = ws4[0] * relu(acc[0]);
    part = fmaf(ws4[1], relu(acc[1]), part);
    part = fmaf(ws4[2], relu(acc[2]), part);
    part = fmaf(ws4[3], relu(acc[3]), part);
    return part;
}
__device__ __forceinline__ float pair_score(float part, float ksc) {
    return (part + __shfl_xor(part, 16, 64)) * ksc;
}

}  // namespace
}  // namespace dsa
