// Sparse MLA attention in MHA mode on gfx950.
//
// Method: the DeepSeek-V3.2 paper's section list (page aipaper.jasonlin.tech,
// "Sections") names the two modes of MLA ("Appendix A MHA and MQA Modes of
// MLA"); DSA itself runs in MQA mode ("Paper Breakdown: DeepSeek-V3.2",
// section 2 "DSA under MLA (MQA Mode)").  In MHA mode every head attends
// over its own keys and values, up-projected from the same latent entries
// c_s (512 latent + 64 rope):
//     key of token s, head h   = [W_UK[h] c_s[:512] ; c_s[512:]]   (192)
//     value of token s, head h = W_UV[h] c_s[:512]                 (128)
// with per-head queries [q_nope ; q_rope] (192).
//
// Two kernels:
//  * mha_up_project: the per-head key and value parts that depend on the head
//    (W_UK[h] c_s[:512], W_UV[h] c_s[:512]) of every latent row into the
//    workspace (bf16, fp32 accumulation), a dense contraction on bf16 MFMA:
//    out^T[col, token] = W[col, :] . c[token, :512] for the 256 output
//    columns (128 key + 128 value) of one head and 64 tokens per workgroup.
//    The rope part of the key is one part shared by every head: it is read
//    from the latent row itself.
//  * sparse_mha_attn: one workgroup per query token, 16 waves x 8 heads, 8
//    lanes per head.  Each selected token's key block ([128 heads][128],
//    32 KiB) and value block ([128][128], 32 KiB) are contiguous, so a wave
//    reads 2 KiB + 2 KiB per token in 16-byte pieces, plus the token's
//    128-byte rope part, which all heads read; a head's dot product is split
//    over its 8 lanes (16 head key dims and 8 rope dims each) and reduced
//    across them.  Online softmax in base 2 per head, fp32 accumulators, bf16
//    output.  Every gathered per-head element is used once (no head shares
//    it), so the kernel is bound by memory, not by arithmetic.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int H = 128, DC = 512, DR = 64, DN = 128, DVH = 128;
constexpr int DK = DN + DR;       // 192: key / query width per head
constexpr int LAT_ROW = DC + DR;  // 576: latent entry width

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---------------------------------------------------------------------------
// Up-projection: 256 threads, 64 latent rows x (one head's 256 output columns).
// Wave w: columns 64*(w&1) .. +63 of the key part (w < 2, W = W_UK[h]) or of
// the value part (w >= 2, W = W_UV[h]).  Per 32-wide k step a wave does 4 x 4
// MFMAs (column blocks x token blocks) on fragments loaded from global memory
// (the 64 rows' latent tile is shared by the four waves through the caches).
constexpr int UP_ROWS = 64;
constexpr int UP_PITCH = 64 + 8;  // LDS staging row: 64 bf16 + 16 bytes pad

__global__ __launch_bounds__(256) void mha_up_project(const uint16_t* __restrict__ kv,
                                                      const uint16_t* __restrict__ w_uk,
                                                      const uint16_t* __restrict__ w_uv,
                                                      uint16_t* __restrict__ kh,
                                                      uint16_t* __restrict__ vh, long long rows) {
    __shared__ __attribute__((aligned(16))) uint16_t stage[4][UP_ROWS * UP_PITCH];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, g = lane >> 4;
    const int h = blockIdx.y;
    const long long r0 = (long long)blockIdx.x * UP_ROWS;
    const uint16_t* __restrict__ W = (wave < 2 ? w_uk : w_uv) + (size_t)h * 128 * DC;
    const int col0 = 64 * (wave & 1);

    f32x4 acc[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[cb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this lane's rows: weights row col0 + 16 cb + m, latent rows r0 + 16 tb + m
    const uint16_t* wrow[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) wrow[cb] = W + (size_t)(col0 + 16 * cb + m) * DC + 8 * g;
    const uint16_t* crow[4];
    bool cvalid[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const long long r = r0 + 16 * tb + m;
        cvalid[tb] = r < rows;
        crow[tb] = kv + (size_t)(cvalid[tb] ? r : 0) * LAT_ROW + 8 * g;
    }
#pragma unroll 2
    for (int ks = 0; ks < DC / 32; ++ks) {
        bf16x8_t a[4], b[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            a[cb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(wrow[cb] + 32 * ks));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            uint4 x = *reinterpret_cast<const uint4*>(crow[tb] + 32 * ks);
            if (!cvalid[tb]) x = uint4{0u, 0u, 0u, 0u};
            b[tb] = __builtin_bit_cast(bf16x8_t, x);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[cb][tb] = mfma16(a[cb], b[tb], acc[cb][tb]);
    }

    // acc[cb][tb] lane (m, g): out^T[col 16cb + 4g + i][token 16tb + m].
    // Stage as [token][64 columns] bf16, then store 16-byte row pieces.
    uint16_t* st = stage[wave];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const uint32_t lo = (uint32_t)bf16_bits(acc[cb][tb][0]) | ((uint32_t)bf16_bits(acc[cb][tb][1]) << 16);
            const uint32_t hi = (uint32_t)bf16_bits(acc[cb][tb][2]) | ((uint32_t)bf16_bits(acc[cb][tb][3]) << 16);
            *reinterpret_cast<uint2*>(st + (16 * tb + m) * UP_PITCH + 16 * cb + 4 * g) = uint2{lo, hi};
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int c = it * 64 + lane;  // 16-byte piece: token c / 8, columns 8 * (c % 8)
        const int tok = c >> 3, pc = c & 7;
        const long long r = r0 + tok;
        if (r < rows) {
            const uint4 x = *reinterpret_cast<const uint4*>(st + tok * UP_PITCH + 8 * pc);
            uint16_t* dst = wave < 2 ? kh + ((size_t)r * H + h) * DN + col0 + 8 * pc
                                     : vh + ((size_t)r * H + h) * DVH + col0 + 8 * pc;
            *reinterpret_cast<uint4*>(dst) = x;
        }
    }
}

// ---------------------------------------------------------------------------
// Attention over per-head keys and values: 1024 threads per query token.
constexpr int AT = 1024;
constexpr int SLOTS = 2048;
constexpr int TILE = 2;  // selected tokens loaded per step

__device__ __forceinline__ void bf16x8_to_f32(const uint4& x, float* f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__global__ __launch_bounds__(AT) void sparse_mha_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ kh,
    const uint16_t* __restrict__ vh, const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
    float* __restrict__ lse, int T, int N, int k, float scale_log2) {
    __shared__ int32_t sidx[SLOTS];
    __shared__ int s_n;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hh = lane >> 3, p = lane & 7;
    const int h = 8 * wave + hh;
    const size_t row = blockIdx.x;
    const int b = (int)(row / (unsigned)T);

    // the row's valid slots, in slot order, compacted into LDS with a
    // block-wide prefix sum (slot order keeps runs reproducible)
    __shared__ int wsum[AT / 64];
    {
        int total = 0;
        for (int i0 = 0; i0 < k; i0 += AT) {
            const int i = i0 + tid;
            const int s = i < k ? idx[row * k + i] : -1;
            const bool ok = s >= 0 && s < N;
            const unsigned long long bal = __ballot(ok);
            if (lane == 0) wsum[wave] = __popcll(bal);
            __syncthreads();
            int before = 0, all = 0;
#pragma unroll
            for (int w = 0; w < AT / 64; ++w) {
                before += w < wave ? wsum[w] : 0;
                all += wsum[w];
            }
            __syncthreads();
            if (ok) sidx[total + before + __popcll(bal & ((1ull << lane) - 1ull))] = s;
            total += all;
        }
        if (tid == 0) s_n = total;
    }
    __syncthreads();
    const int n = s_n;

    // this lane's 24 query dims of head h: head key dims 16p .. 16p+15 and
    // rope dims 8p .. 8p+7
    float qf[24];
    {
        const uint16_t* qp = q + (row * H + h) * DK;
#pragma unroll
        for (int j = 0; j < 2; ++j) bf16x8_to_f32(*reinterpret_cast<const uint4*>(qp + 16 * p + 8 * j), qf + 8 * j);
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(qp + DN + 8 * p), qf + 16);
    }
    const uint16_t* kb = kh + ((size_t)b * N * H + h) * DN + 16 * p;
    const uint16_t* rb = kv + (size_t)b * N * LAT_ROW + DC + 8 * p;
    const uint16_t* vb = vh + ((size_t)b * N * H + h) * DVH + 16 * p;
    const size_t kstride = (size_t)H * DN, vstride = (size_t)H * DVH;

    float o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) o[j] = 0.f;
    float m_run = -__builtin_inff(), l_run = 0.f;

    for (int i = 0; i < n; i += TILE) {
        uint4 kx[TILE][3], vx[TILE][2];
        bool ok[TILE];
#pragma unroll
        for (int j = 0; j < TILE; ++j) {
            ok[j] = i + j < n;
            const int s = ok[j] ? sidx[i + j] : sidx[i];
            const uint16_t* kp = kb + (size_t)s * kstride;
            const uint16_t* vp = vb + (size_t)s * vstride;
#pragma unroll
            for (int c = 0; c < 2; ++c) kx[j][c] = *reinterpret_cast<const uint4*>(kp + 8 * c);
            kx[j][2] = *reinterpret_cast<const uint4*>(rb + (size_t)s * LAT_ROW);
#pragma unroll
            for (int c = 0; c < 2; ++c) vx[j][c] = *reinterpret_cast<const uint4*>(vp + 8 * c);
        }
        float x[TILE];
#pragma unroll
        for (int j = 0; j < TILE; ++j) {
            float kf[24];
#pragma unroll
            for (int c = 0; c < 3; ++c) bf16x8_to_f32(kx[j][c], kf + 8 * c);
            float z = 0.f;
#pragma unroll
            for (int d = 0; d < 24; ++d) z = fmaf(qf[d], kf[d], z);
            z += __shfl_xor(z, 1, 64);
            z += __shfl_xor(z, 2, 64);
            z += __shfl_xor(z, 4, 64);
            x[j] = ok[j] ? z * scale_log2 : -__builtin_inff();
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < TILE; ++j) mx = fmaxf(mx, x[j]);
        if (mx > m_run) {  // a new running max: rescale what has been summed
            const float f = __builtin_amdgcn_exp2f(m_run - mx);
            l_run *= f;
#pragma unroll
            for (int d = 0; d < 16; ++d) o[d] *= f;
            m_run = mx;
        }
#pragma unroll
        for (int j = 0; j < TILE; ++j) {
            const float pj = __builtin_amdgcn_exp2f(x[j] - m_run);
            l_run += pj;
            float vf[16];
            bf16x8_to_f32(vx[j][0], vf);
            bf16x8_to_f32(vx[j][1], vf + 8);
#pragma unroll
            for (int d = 0; d < 16; ++d) o[d] = fmaf(pj, vf[d], o[d]);
        }
    }

    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int d = 0; d < 8; ++d)
        pk[d] = (uint32_t)bf16_bits(o[2 * d] * inv) | ((uint32_t)bf16_bits(o[2 * d + 1] * inv) << 16);
    uint16_t* op = out + (row * H + h) * DVH + 16 * p;
    *reinterpret_cast<uint4*>(op) = uint4{pk[0], pk[1], pk[2], pk[3]};
    *reinterpret_cast<uint4*>(op + 8) = uint4{pk[4], pk[5], pk[6], pk[7]};
    if (lse != nullptr && p == 0)
        lse[row * H + h] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -__builtin_inff();
}

}  // namespace

size_t attn_mha_workspace_bytes(int B, int N) {
    const size_t rows = (size_t)B * N;
    return align_up(rows * H * DN * sizeof(uint16_t)) + align_up(rows * H * DVH * sizeof(uint16_t));
}

dsa_status launch_attn_mha_bf16(const void* q, const void* kv, const void* w_uk, const void* w_uv,
                                const int32_t* idx, void* out, float* lse, int B, int T, int N,
                                int k, float sm_scale, void* workspace, hipStream_t stream) {
    if (k > SLOTS) return DSA_ERR_UNSUPPORTED;
    const long long rows_kv = (long long)B * N;
    const long long rows_q = (long long)B * T;
    if (rows_q > 0x7fffffffLL || (rows_kv + UP_ROWS - 1) / UP_ROWS > 0x7fffffffLL)
        return DSA_ERR_UNSUPPORTED;
    auto* kh = static_cast<uint16_t*>(workspace);
    auto* vh = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                           align_up((size_t)rows_kv * H * DN * sizeof(uint16_t)));
    DSA_TIMED("mha_up_project", stream,
              mha_up_project<<<dim3((unsigned)((rows_kv + UP_ROWS - 1) / UP_ROWS), H), 256, 0,
                               stream>>>(static_cast<const uint16_t*>(kv),
                                         static_cast<const uint16_t*>(w_uk),
                                         static_cast<const uint16_t*>(w_uv), kh, vh, rows_kv));
    dsa_status st = launch_status();
    if (st != DSA_OK) return st;
    DSA_TIMED("sparse_mha_attn", stream,
              sparse_mha_attn<<<dim3((unsigned)rows_q), AT, 0, stream>>>(
                  static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), kh, vh, idx,
                  static_cast<uint16_t*>(out), lse, T, N, k, sm_scale * kLog2e));
    return launch_status();
}

}  // namespace dsa
