// Cache append on gfx950: the step before the path at decode.
//
// Each selected token contributes its latent entry c_s and each candidate its
// indexer key, held per token; the indexer runs in FP8 ("Paper Breakdown:
// DeepSeek-V3.2", section 2 "Architecture: DSA (§2.1)", the index-score
// formula and the FP8 note under it).  New token t of sequence b goes to
// cache row pos[b] + t: its indexer key (float32) is quantised to e4m3fn
// codes with one float32 scale per token, scale = amax / 448 (1 for a row of
// zeros), code = round-to-nearest-even(clamp(x / scale, +-448)); its latent
// row is copied unchanged.  Rows whose position falls outside [0, N) are
// dropped.
//
// One wave per new token.  The key row (128 floats) sits two elements per
// lane: a butterfly max over the wave gives amax, both divisions are IEEE
// float32 divisions (correctly rounded), and v_cvt_pk_fp8_f32 rounds a pair
// of quotients to OCP e4m3fn codes, stored as one 16-bit word per lane.  The
// latent row is copied with 16-byte loads and stores.  HBM-bound: 132 + the
// latent row's bytes written and 512 + those bytes read per token.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int CT = 256;          // threads per workgroup: four rows
constexpr float kE4M3Max = 448.f;

// Copy one row of `bytes` bytes (16-byte aligned, bytes % 16 == 0 when vec).
__device__ __forceinline__ void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                         int bytes, bool vec, int lane) {
    if (vec) {
        for (int c = lane; c < bytes / 16; c += 64)
            reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
    } else {
        for (int c = lane; c < bytes / 4; c += 64)
            reinterpret_cast<uint32_t*>(dst)[c] = reinterpret_cast<const uint32_t*>(src)[c];
    }
}

template <bool FP8>
__global__ __launch_bounds__(CT) void cache_append_kernel(
    const float* __restrict__ k_new, const uint8_t* __restrict__ kv_new, uint8_t* __restrict__ k_cache,
    float* __restrict__ k_scale, uint8_t* __restrict__ kv_cache, const int32_t* __restrict__ pos, int B,
    int T, int N, int d_i, int kv_row_bytes) {
    const int lane = threadIdx.x & 63;
    const long long r = (long long)blockIdx.x * (CT / 64) + (threadIdx.x >> 6);  // b * T + t
    if (r >= (long long)B * T) return;
    const int b = (int)(r / T), t = (int)(r % T);
    const long long p = (long long)pos[b] + t;
    if (p < 0 || p >= N) return;
    const size_t dst_row = (size_t)b * N + (size_t)p;

    if (FP8) {
        // d_i == 128: elements 2*lane and 2*lane + 1
        const float2 x = reinterpret_cast<const float2*>(k_new + r * 128)[lane];
        float a = fmaxf(fabsf(x.x), fabsf(x.y));
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
        const float scale = a > 0.f ? a / kE4M3Max : 1.f;
        const float y0 = fminf(fmaxf(x.x / scale, -kE4M3Max), kE4M3Max);
        const float y1 = fminf(fmaxf(x.y / scale, -kE4M3Max), kE4M3Max);
        const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        reinterpret_cast<uint16_t*>(k_cache + dst_row * 128)[lane] = (uint16_t)(packed & 0xffff);
        if (lane == 0) k_scale[dst_row] = scale;
    } else {
        const float* src = k_new + r * d_i;
        float* dst = reinterpret_cast<float*>(k_cache) + dst_row * d_i;
        for (int j = lane; j < d_i; j += 64) dst[j] = src[j];
    }
    copy_row(kv_new + r * kv_row_bytes, kv_cache + dst_row * kv_row_bytes, kv_row_bytes,
             (kv_row_bytes & 15) == 0, lane);
}

}  // namespace

dsa_status launch_cache_append(const float* k_new, const void* kv_new, void* k_cache, float* k_scale,
                               void* kv_cache, const int32_t* pos, int B, int T, int N, int d_i,
                               int kv_row_bytes, bool fp8, hipStream_t stream) {
    const long long rows = (long long)B * T;
    const unsigned grid = (unsigned)((rows + CT / 64 - 1) / (CT / 64));
    auto args = [&](auto kern, const char* name) {
        DSA_TIMED(name, stream,
                  kern<<<grid, CT, 0, stream>>>(k_new, static_cast<const uint8_t*>(kv_new),
                                                static_cast<uint8_t*>(k_cache), k_scale,
                                                static_cast<uint8_t*>(kv_cache), pos, B, T, N, d_i,
                                                kv_row_bytes));
    };
    if (fp8) args(cache_append_kernel<true>, "cache_append_kernel<true>");
    else args(cache_append_kernel<false>, "cache_append_kernel<false>");
    return launch_status();
}

}  // namespace dsa
