// Lightning-indexer scores on gfx950.
//
// Formula ("Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture: DSA
// (§2.1)"): I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]), one key per token
// shared by the H_I = 8 indexer heads, FP8 operands.
//
// FP8 path.  The contraction over d_I = 128 is exactly one
// v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3 -> fp32).  The 16 MFMA rows are
// (4 queries x 4 heads); two MFMAs (heads 0-3 and 4-7) put all 8 head dots
// of one (query, key) pair in the same lane, so ReLU, the (w * q_scale)
// weighted head sum and the key scale run in registers with no cross-lane
// traffic.
//
//  * indexer_fp8_tiled  (T >= 16): a workgroup owns 64 queries (8 waves x 8)
//    and a range of keys; 64-key tiles are staged through LDS (rows padded
//    to 144 B so the 16 lanes that read one 32-byte slice of 16 different
//    keys hit distinct banks) and double-buffered: the next tile's global
//    loads are in flight while the current tile is multiplied.  Each wave
//    collects its 8 x 64 scores in LDS and writes them as whole 256-byte row
//    segments with 16-byte stores.
//  * indexer_fp8_stream (T < 16, e.g. decode): the key stream is read once,
//    so each wave loads its 16-key fragments straight from HBM (see the
//    kernel for its own MFMA row layout and store pattern).
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int HI = 8;      // indexer heads
constexpr int DI = 128;    // indexer dim = bytes per FP8 row
constexpr int NT = 256;    // threads per workgroup (4 waves)

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

__device__ void fill_neg_inf(float* __restrict__ out_b, int t0, int t1, int N, int s0, int s1) {
    const float ninf = -__builtin_inff();
    for (int t = t0; t < t1; ++t)
        for (int s = s0 + (int)threadIdx.x; s < s1; s += (int)blockDim.x) out_b[(size_t)t * N + s] = ninf;
}

// ---------------------------------------------------------------------------
constexpr int TQB = 64;     // queries per workgroup (tiled)
constexpr int TILE = 64;    // keys per LDS tile
constexpr int ROWB = 144;   // LDS bytes per key row (128 + 16 pad)

constexpr int OST = 80;     // LDS floats per staged output row (64 + 16: rows 16 banks apart)
constexpr int NTT = 512;    // threads of the tiled kernel: 8 waves x 8 queries
constexpr int QPW = TQB / (NTT / 64);   // queries per wave
constexpr int GPW = QPW / 4;            // 4-query MFMA groups per wave

template <bool FILL>
__global__ __launch_bounds__(NTT) void indexer_fp8_tiled(
    const uint8_t* __restrict__ q, const float* __restrict__ qs, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const float* __restrict__ w, float* __restrict__ scores,
    int T, int N, int q_offset, int keys_per_wg) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][TILE * ROWB];
    __shared__ float lds_ks[2][TILE];
    __shared__ __attribute__((aligned(16))) float lds_o[NTT / 64][QPW * OST];

    const int b = blockIdx.z;
    const int t0 = blockIdx.x * TQB;
    const int s_begin = blockIdx.y * keys_per_wg;
    const int s_end = min(N, s_begin + keys_per_wg);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, kb = lane >> 4;
    const int t_end = min(T, t0 + TQB);
    const int s_vis = min(s_end, q_offset + t_end);  // keys [s_begin, s_vis) are visible to some query
    const size_t row0 = (size_t)b * T;
    float* __restrict__ out_b = scores + row0 * N;
    const uint8_t* __restrict__ k_b = k + (size_t)b * N * DI;
    const float* __restrict__ ks_b = ks + (size_t)b * N;
    // whole 16-byte output chunks: rows start 16-byte aligned, ranges end on 4
    const bool vec_out = (N & 3) == 0;

    const int n_tiles = s_vis > s_begin ? (s_vis - s_begin + TILE - 1) / TILE : 0;
    if (n_tiles > 0) {
        const int tw0 = t0 + QPW * wave;
        i32x8 a[GPW][2];
        float ws[GPW][HI];
#pragma unroll
        for (int g = 0; g < GPW; ++g) load_queries(q, qs, w, row0, tw0 + 4 * g, T, lane, a[g], ws[g]);
        float* ost = lds_o[wave];

        // cooperative staging: 512 16-byte chunks per tile, one per thread
        const int c_key = tid >> 3, c_piece = tid & 7;
        uint4 r0;
        float rks = 0.f;
        auto fetch = [&](int s0) {
            const uint4 zero = {0u, 0u, 0u, 0u};
            const int s_a = s0 + c_key;
            r0 = s_a < N ? *reinterpret_cast<const uint4*>(k_b + (size_t)s_a * DI + 16 * c_piece) : zero;
            if (tid < TILE) rks = (s0 + tid) < N ? ks_b[s0 + tid] : 0.f;
        };
        auto stage = [&](int buf) {
            *reinterpret_cast<uint4*>(&lds_k[buf][c_key * ROWB + 16 * c_piece]) = r0;
            if (tid < TILE) lds_ks[buf][tid] = rks;
        };

        fetch(s_begin);
        stage(0);
        __syncthreads();
        for (int it = 0; it < n_tiles; ++it) {
            const int s0 = s_begin + it * TILE;
            const int buf = it & 1;
            const bool more = it + 1 < n_tiles;
            if (more) fetch(s0 + TILE);
            if (tw0 < t_end) {
                // a clean tile: every key visible to all of the wave's queries, all in range
                const bool clean = vec_out && s0 + TILE - 1 <= q_offset + tw0 && tw0 + QPW <= T &&
                                   s0 + TILE <= s_end;
#pragma unroll
                for (int sub = 0; sub < TILE / 16; ++sub) {
                    const int key = 16 * sub + m;
                    const uint8_t* src = &lds_k[buf][key * ROWB + 32 * kb];
                    const i32x8 bf = pack8(*reinterpret_cast<const uint4*>(src),
                                           *reinterpret_cast<const uint4*>(src + 16));
                    const float ksc = lds_ks[buf][key];
                    const int s_abs = s0 + key;
                    f32x4 acc[GPW][2];
#pragma unroll
                    for (int g = 0; g < GPW; ++g) {
                        acc[g][0] = mfma_fp8(a[g][0], bf);
                        acc[g][1] = mfma_fp8(a[g][1], bf);
                    }
#pragma unroll
                    for (int g = 0; g < GPW; ++g) {
                        float sc = head_sum(acc[g][0], acc[g][1], ws[g]) * ksc;
                        if (!clean && s_abs > q_offset + tw0 + 4 * g + kb) sc = -__builtin_inff();
                        ost[(4 * g + kb) * OST + key] = sc;
                    }
                }
                // QPW rows x 64 keys out of LDS: lane l takes 16 bytes of row
                // 4j + l/16 per step, each row a whole 256-byte segment
                const int c = lane & 15;
#pragma unroll
                for (int j = 0; j < QPW / 4; ++j) {
                    const int r = 4 * j + (lane >> 4);
                    const int t = tw0 + r;
                    const float4 v = *reinterpret_cast<const float4*>(&ost[r * OST + 4 * c]);
                    float* dst = out_b + (size_t)t * N + s0 + 4 * c;
                    if (clean) {
                        *reinterpret_cast<float4*>(dst) = v;
                    } else if (t < T) {
                        if (vec_out) {
                            if (s0 + 4 * c < s_end) *reinterpret_cast<float4*>(dst) = v;
                        } else {
                            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (s0 + 4 * c + e < s_end) dst[e] = vv[e];
                        }
                    }
                }
            }
            if (more) stage(buf ^ 1);
            __syncthreads();
        }
    }
    if (FILL) {
        const int f0 = s_begin + n_tiles * TILE;
        if (f0 < s_end) fill_neg_inf(out_b, t0, t_end, N, f0, s_end);
    }
}

// ---------------------------------------------------------------------------
#ifndef DSA_STREAM_SU
#define DSA_STREAM_SU 8
#endif
#ifndef DSA_STREAM_WG_TARGET
#define DSA_STREAM_WG_TARGET 8192
#endif
constexpr int SU = DSA_STREAM_SU;     // 16-key fragments per wave and block
static_assert(SU % 4 == 0, "fragments are stored in groups of four");

// Stream kernel.  The 16 MFMA rows are (2 queries x 8 heads), one MFMA per
// query pair and 16 keys; C lane l holds rows 4*(l/16)+i, i.e. query l/32 of
// the pair, heads 4*((l/16)&1)+i, and key l%16, so the two head halves of a
// score meet with one lane exchange (l ^ 16).  NP query pairs per workgroup.
//
// Each wave walks blocks of 16*SU consecutive keys (the four waves take
// turns); the scores of 64 consecutive keys are gathered across lanes into
// one 256-byte store per query.  Key loads are unconditional (addresses
// clamped into the visible range; values past it are never stored unmasked)
// and the next block's loads are issued before this block's stores.
template <bool FILL, int NP>
__global__ __launch_bounds__(NT) void indexer_fp8_stream(
    const uint8_t* __restrict__ q, const float* __restrict__ qs, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const float* __restrict__ w, float* __restrict__ scores,
    int T, int N, int q_offset, int keys_per_wg) {
    constexpr int SQ = 2 * NP;
    const int b = blockIdx.z;
    const int tq0 = blockIdx.y * SQ;
    const int s_begin = blockIdx.x * keys_per_wg;
    const int s_end = min(N, s_begin + keys_per_wg);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, kb = lane >> 4;
    const int t_end = min(T, tq0 + SQ);
    const int s_vis = min(s_end, q_offset + t_end);
    const size_t row0 = (size_t)b * T;
    float* __restrict__ out_b = scores + row0 * N;
    const uint8_t* __restrict__ k_b = k + (size_t)b * N * DI;
    const float* __restrict__ ks_b = ks + (size_t)b * N;

    // A rows m: query tq0 + 2p + (m >> 3), head m & 7
    i32x8 a[NP];
    float ws[NP][4];
    int tl[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int ta = tq0 + 2 * p + (m >> 3), h = m & 7;
        if (ta < T) {
            const uint4* src = reinterpret_cast<const uint4*>(q + ((row0 + ta) * HI + h) * DI + 32 * kb);
            a[p] = pack8(src[0], src[1]);
        } else {
            a[p] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        tl[p] = tq0 + 2 * p + (kb >> 1);  // the query this lane's C rows belong to
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h2 = 4 * (kb & 1) + i;
            ws[p][i] = tl[p] < T ? w[(row0 + tl[p]) * HI + h2] * qs[(row0 + tl[p]) * HI + h2] : 0.f;
        }
    }

    uint4 x0[SU], x1[SU];
    float kss[SU];
    auto load = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int s = min(base + 16 * u + m, s_vis - 1);
            const uint4* p = reinterpret_cast<const uint4*>(k_b + (size_t)s * DI + 32 * kb);
            x0[u] = p[0];
            x1[u] = p[1];
            kss[u] = ks_b[s];
        }
    };
    float sc[NP][SU];
    auto comp = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const i32x8 bf = pack8(x0[u], x1[u]);
            const int s_abs = base + 16 * u + m;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const f32x4 acc = mfma_fp8(a[p], bf);
                float part = ws[p][0] * relu(acc[0]);
                part = fmaf(ws[p][1], relu(acc[1]), part);
                part = fmaf(ws[p][2], relu(acc[2]), part);
                part = fmaf(ws[p][3], relu(acc[3]), part);
                float v = (part + __shfl_xor(part, 16, 64)) * kss[u];
                if (s_abs > q_offset + tl[p]) v = -__builtin_inff();
                sc[p][u] = v;
            }
        }
    };
    // lane l of group g stores key base + 64g + l: fragment 4g + l/16, key
    // l%16, read from lane l%16 (first query of the pair) or 32 + l%16
    auto store = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < SU / 4; ++g) {
            const int key = base + 64 * g + lane;
            const bool in = (key & ~15) < s_vis && key < s_end;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    const int tq = tq0 + 2 * p + qq;
                    float v = 0.f;
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const float x = __shfl(sc[p][4 * g + f], 32 * qq + m, 64);
                        v = kb == f ? x : v;
                    }
                    if (in && tq < t_end) out_b[(size_t)tq * N + key] = v;
                }
            }
        }
    };
    int base = s_begin + 16 * SU * wave;
    if (base < s_vis) load(base);
    for (; base < s_vis; base += 64 * SU) {
        comp(base);
        if (base + 64 * SU < s_vis) load(base + 64 * SU);
        store(base);
    }
    if (FILL) {
        // fragments cover [s_begin, s_vis) rounded up to 16; fill the rest
        const int f0 = s_begin + ((max(s_vis - s_begin, 0) + 15) / 16) * 16;
        if (f0 < s_end) fill_neg_inf(out_b, tq0, t_end, N, f0, s_end);
    }
}

// ---------------------------------------------------------------------------
// fp32 reference-precision path (small head counts and dims): one thread per
// (query, key), the query row in LDS.
constexpr int F32_MAX_HD = 4096;

__global__ __launch_bounds__(NT) void indexer_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ w,
    float* __restrict__ scores, int T, int N, int H_I, int d_I, int q_offset, int fill) {
    __shared__ float qrow[F32_MAX_HD];
    __shared__ float wrow[16];
    const int b = blockIdx.z, t = blockIdx.y;
    const size_t row = (size_t)b * T + t;
    for (int i = threadIdx.x; i < H_I * d_I; i += NT) qrow[i] = q[row * H_I * d_I + i];
    if (threadIdx.x < H_I) wrow[threadIdx.x] = w[row * H_I + threadIdx.x];
    __syncthreads();
    const int s = blockIdx.x * NT + threadIdx.x;
    if (s >= N) return;
    float* dst = scores + row * N + s;
    if (s > q_offset + t) {
        if (fill) *dst = -__builtin_inff();
        return;
    }
    const float* kr = k + ((size_t)b * N + s) * d_I;
    float acc = 0.f;
    for (int j = 0; j < H_I; ++j) {
        float dot = 0.f;
        for (int d = 0; d < d_I; ++d) dot = fmaf(qrow[j * d_I + d], kr[d], dot);
        acc = fmaf(wrow[j], fmaxf(dot, 0.f), acc);
    }
    *dst = acc;
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

dsa_status launch_indexer_fp8(const uint8_t* q, const float* qs, const uint8_t* k,
                              const float* ks, const float* w, float* scores,
                              int B, int T, int N, int q_offset, bool fill_masked,
                              hipStream_t stream) {
    const long long n_vis = fill_masked ? N : std::min<long long>(N, (long long)q_offset + T);
    if (T >= 16) {
        const int nqb = ceil_div(T, TQB);
        // aim for >= 2048 workgroups; key ranges are whole tiles, 256..8192 keys
        long long kpw = (long long)nqb * B * n_vis / 2048;
        kpw = std::max<long long>(256, std::min<long long>(8192, kpw));
        kpw = (kpw + TILE - 1) / TILE * TILE;
        dim3 grid(nqb, ceil_div(n_vis, kpw), B);
        if (fill_masked)
            indexer_fp8_tiled<true><<<grid, NTT, 0, stream>>>(q, qs, k, ks, w, scores, T, N, q_offset, (int)kpw);
        else
            indexer_fp8_tiled<false><<<grid, NTT, 0, stream>>>(q, qs, k, ks, w, scores, T, N, q_offset, (int)kpw);
        return launch_status();
    }
    const int np = T <= 2 ? 1 : 2;
    const int nqg = ceil_div(T, 2 * np);
    long long kpw = (long long)nqg * B * n_vis / DSA_STREAM_WG_TARGET;
    kpw = std::max<long long>(1024, std::min<long long>(16384, kpw));
    kpw = (kpw + 64 * SU - 1) / (64 * SU) * (64 * SU);
    dim3 grid(ceil_div(n_vis, kpw), nqg, B);
    auto go = [&](auto kern) {
        kern<<<grid, NT, 0, stream>>>(q, qs, k, ks, w, scores, T, N, q_offset, (int)kpw);
    };
    if (np == 1) {
        if (fill_masked) go(indexer_fp8_stream<true, 1>); else go(indexer_fp8_stream<false, 1>);
    } else {
        if (fill_masked) go(indexer_fp8_stream<true, 2>); else go(indexer_fp8_stream<false, 2>);
    }
    return launch_status();
}

dsa_status launch_indexer_f32(const float* q, const float* k, const float* w, float* scores,
                              int B, int T, int N, int H_I, int d_I, int q_offset,
                              bool fill_masked, hipStream_t stream) {
    if (H_I * d_I > F32_MAX_HD || H_I > 16) return DSA_ERR_UNSUPPORTED;
    dim3 grid(ceil_div(N, NT), T, B);
    indexer_f32_kernel<<<grid, NT, 0, stream>>>(q, k, w, scores, T, N, H_I, d_I, q_offset,
                                                fill_masked ? 1 : 0);
    return launch_status();
}

}  // namespace dsa
