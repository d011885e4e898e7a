// Sparse MLA attention in MQA mode on gfx950.
//
// Method ("Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture: DSA
// (§2.1)"): u_t = Attn(h_t, {c_s : I[t,s] in Top-k(I[t,:])}); under "DSA
// under MLA (MQA Mode)" one latent vector c_s (576 wide: 512 latent + 64
// rope) per selected token is shared by all 128 query heads, and the value
// is its 512-wide latent part.
//
// bf16 path: one workgroup (8 waves, 16 heads each) per query token and
// slot range.  Per 32-key tile the selected rows are gathered with 16-byte
// coalesced loads (a row is 72 chunks: 64 latent + 8 rope) and written to
// LDS twice: row-major for the key product, and with the latent part
// transposed (V^T, keys contiguous) for the value product, the transpose
// done in registers on 4x8 blocks.  Tiles are double-buffered: the next
// tile's gather is in flight while the current one is multiplied.
//
// Per wave and tile:
//   S^T[key, head] = K[key, :] . Q[head, :]        18 x 2 bf16 MFMA 16x16x32
//     (A = key rows from LDS, B = the wave's 16 query heads kept in VGPRs;
//      computing S^T instead of S puts one head per lane column, which is
//      exactly the row layout the P operand of the value product needs)
//   online softmax in base 2 with a lazy rescale (the running reference
//     max only moves when a tile max exceeds it by more than 8, so exp2
//     stays <= 256 and the O rescale is rare)
//   O[head, v] += P[head, key] V[key, v]           32 bf16 MFMA 16x16x32
//     (the key order inside the MFMA's K dimension is permuted to match
//      the accumulator layout of S^T; V^T is read with the same permutation)
// The O accumulator (16 heads x 512 fp32) stays in registers.  Decode-sized
// batches split the slots over several workgroups and merge the partial
// (O, max, sum) triples in attn_combine.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int H = 128, DQK = 576, DV = 512;
constexpr int NWV = 8;                   // waves per workgroup, 16 heads each
constexpr int NTA = NWV * 64;            // 512 threads
constexpr int TK = 32;                   // keys per tile
constexpr int KROW = DQK * 2 + 16;       // LDS bytes per key row (padded)
constexpr int VROW = TK * 2 + 8;         // LDS bytes per V^T row (padded)
constexpr int KBUF = TK * KROW;          // 37376 B
constexpr int VBUF = DV * VROW;          // 36864 B
constexpr int SLOTS = 2048;              // max index slots per workgroup
constexpr float RESCALE_GAP = 8.0f;      // lazy rescale threshold (log2 units)

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& x) {
    return __builtin_bit_cast(bf16x8, x);
}

__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

template <bool PARTIAL>
__global__ __launch_bounds__(NTA) void sparse_mla_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int T, int N, int k, int slots_per_split, float scale_log2) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (KBUF + VBUF)];
    __shared__ int32_t sidx[SLOTS];
    __shared__ int s_last;

    const int split = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
    const int nsplit = gridDim.x;
    const size_t row = (size_t)b * T + t;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, g = lane >> 4;
    const int slot0 = split * slots_per_split;
    const int nslots = max(0, min(k - slot0, slots_per_split));
    const uint16_t* __restrict__ kv_b = kv + (size_t)b * N * DQK;

    // ---- slot indices of this workgroup; find the last valid one
    if (tid == 0) s_last = -1;
    __syncthreads();
    int my_last = -1;
    for (int i = tid; i < nslots; i += NTA) {
        const int id = idx[row * k + slot0 + i];
        sidx[i] = id;
        if (id >= 0 && id < N) my_last = i;
    }
    if (my_last >= 0) atomicMax(&s_last, my_last);

    // ---- this wave's 16 query heads, kept as B operands (k = 8*(l/16)+j)
    bf16x8 qf[DQK / 32];
    {
        const uint16_t* qh = q + (row * H + 16 * wave + m) * DQK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < DQK / 32; ++ks)
            qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qh + 32 * ks));
    }
    __syncthreads();
    const int n_tiles = (s_last + TK) / TK;  // 0 when no slot is valid

    f32x4 o[DV / 16];
#pragma unroll
    for (int i = 0; i < DV / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -__builtin_inff();  // running reference max of head m (log2 units)
    float l_part = 0.f;               // this lane's part of head m's exp-sum

    // gather roles: latent chunk c (8 columns) of keys 4*kg..4*kg+3; rope
    // chunk rc of key rk (threads < 256)
    const int c = tid & 63, kg = tid >> 6;
    const int rk = tid >> 3, rc = 64 + (tid & 7);
    uint4 lat[4], rope;
    auto fetch = [&](int tile) {
        const uint4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sl = tile * TK + 4 * kg + u;
            const int id = sl < nslots ? sidx[sl] : -1;
            lat[u] = (id >= 0 && id < N)
                         ? *reinterpret_cast<const uint4*>(kv_b + (size_t)id * DQK + 8 * c) : zero;
        }
        if (tid < 256) {
            const int sl = tile * TK + rk;
            const int id = sl < nslots ? sidx[sl] : -1;
            rope = (id >= 0 && id < N)
                       ? *reinterpret_cast<const uint4*>(kv_b + (size_t)id * DQK + 8 * rc) : zero;
        }
    };
    auto stage = [&](int buf) {
        uint8_t* kb = lds + buf * (KBUF + VBUF);
        uint8_t* vb = kb + KBUF;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<uint4*>(kb + (4 * kg + u) * KROW + 16 * c) = lat[u];
        if (tid < 256) *reinterpret_cast<uint4*>(kb + rk * KROW + 16 * rc) = rope;
        // V^T: column 8c+j holds keys 4kg..4kg+3 contiguously
        const uint32_t* L0 = reinterpret_cast<const uint32_t*>(&lat[0]);
        const uint32_t* L1 = reinterpret_cast<const uint32_t*>(&lat[1]);
        const uint32_t* L2 = reinterpret_cast<const uint32_t*>(&lat[2]);
        const uint32_t* L3 = reinterpret_cast<const uint32_t*>(&lat[3]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int dw = j >> 1;
            uint2 v;
            if (j & 1) {
                v.x = hi16(L0[dw]) | (L1[dw] & 0xffff0000u);
                v.y = hi16(L2[dw]) | (L3[dw] & 0xffff0000u);
            } else {
                v.x = lo16(L0[dw]) | (L1[dw] << 16);
                v.y = lo16(L2[dw]) | (L3[dw] << 16);
            }
            *reinterpret_cast<uint2*>(vb + (8 * c + j) * VROW + 8 * kg) = v;
        }
    };

    if (n_tiles > 0) {
        fetch(0);
        stage(0);
    }
    __syncthreads();
    for (int it = 0; it < n_tiles; ++it) {
        const int buf = it & 1;
        const bool more = it + 1 < n_tiles;
        if (more) fetch(it + 1);  // in flight while this tile is multiplied
        const uint8_t* kb = lds + buf * (KBUF + VBUF);
        const uint8_t* vb = kb + KBUF;

        // S^T for keys 16*nb + 4*g + i, head m
        f32x4 st[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const uint8_t* kr = kb + (16 * nb + m) * KROW + 16 * g;
#pragma unroll
            for (int ks = 0; ks < DQK / 32; ++ks)
                acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(kr + 64 * ks)), qf[ks], acc);
            st[nb] = acc;
        }
        // validity and tile max of head m
        float x[2][4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = it * TK + 16 * nb + 4 * g + i;
                const int id = sl < nslots ? sidx[sl] : -1;
                const bool ok = id >= 0 && id < N;
                x[nb][i] = ok ? st[nb][i] * scale_log2 : -__builtin_inff();
                mx = fmaxf(mx, x[nb][i]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (__any(mx > m_ref + RESCALE_GAP)) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = exp2f(m_ref - m_new);
            l_part *= alpha;
            float ao[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ao[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
            for (int nv = 0; nv < DV / 16; ++nv)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[nv][i] *= ao[i];
            m_ref = m_new;
        }
        float p[8];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = x[nb][i] == -__builtin_inff() ? 0.f : exp2f(x[nb][i] - m_ref);
                p[4 * nb + i] = e;
                l_part += e;
            }
        const bf16x8 pa = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                           (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        // O += P V, key order {4g..4g+3, 16+4g..16+4g+3} on both operands
#pragma unroll
        for (int nv = 0; nv < DV / 16; ++nv) {
            const uint8_t* vr = vb + (16 * nv + m) * VROW + 8 * g;
            const uint2 v0 = *reinterpret_cast<const uint2*>(vr);
            const uint2 v1 = *reinterpret_cast<const uint2*>(vr + 32);
            const uint4 vv = {v0.x, v0.y, v1.x, v1.y};
            o[nv] = mfma_bf16(pa, as_bf16x8(vv), o[nv]);
        }
        if (more) stage(buf ^ 1);
        __syncthreads();
    }

    // ---- finish: exp-sum of head m over the wave, then per O row
    float l_tot = l_part + __shfl_xor(l_part, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    float lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lo[i] = __shfl(l_tot, 4 * g + i, 64);
    const int h0 = 16 * wave;
    if (PARTIAL) {
        const size_t pbase = (row * nsplit + split) * H;
#pragma unroll
        for (int nv = 0; nv < DV / 16; ++nv)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part_o[(pbase + h0 + 4 * g + i) * DV + 16 * nv + m] = o[nv][i];
        if (g == 0) {
            part_ml[(pbase + h0 + m) * 2 + 0] = m_ref;
            part_ml[(pbase + h0 + m) * 2 + 1] = l_tot;
        }
        return;
    }
    if (lse != nullptr && g == 0)
        lse[row * H + h0 + m] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -__builtin_inff();
    // normalise, stage bf16 rows in LDS (all tile buffers are free now), store 16 B chunks
    uint16_t* ob = reinterpret_cast<uint16_t*>(lds) + wave * 16 * DV;
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = lo[i] > 0.f ? 1.f / lo[i] : 0.f;
#pragma unroll
    for (int nv = 0; nv < DV / 16; ++nv)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ob[(4 * g + i) * DV + 16 * nv + m] = __builtin_bit_cast(uint16_t, (__bf16)(o[nv][i] * inv[i]));
    __syncthreads();
    uint16_t* dst = out + (row * H + h0) * DV;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ch = r * 64 + lane;  // 16-byte chunk of the wave's 16 x 512 block
        *reinterpret_cast<uint4*>(dst + ch * 8) = *reinterpret_cast<const uint4*>(ob + ch * 8);
    }
}

// Merge the per-split (O, max, sum) partials of one query token.
__global__ __launch_bounds__(DV) void attn_combine(const float* __restrict__ part_o,
                                                  const float* __restrict__ part_ml,
                                                  uint16_t* __restrict__ out, float* __restrict__ lse,
                                                  int nsplit) {
    const size_t row = blockIdx.x;
    const int v = threadIdx.x;
    for (int h = 0; h < H; ++h) {
        float M = -__builtin_inff();
        for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((row * nsplit + s) * H + h) * 2]);
        float L = 0.f, acc = 0.f;
        if (M != -__builtin_inff()) {
            for (int s = 0; s < nsplit; ++s) {
                const size_t pb = (row * nsplit + s) * H + h;
                const float ms = part_ml[pb * 2];
                if (ms == -__builtin_inff()) continue;
                const float f = exp2f(ms - M);
                L += part_ml[pb * 2 + 1] * f;
                acc += part_o[pb * DV + v] * f;
            }
        }
        const float o = L > 0.f ? acc / L : 0.f;
        out[(row * H + h) * DV + v] = __builtin_bit_cast(uint16_t, (__bf16)o);
        if (lse != nullptr && v == 0) lse[row * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -__builtin_inff();
    }
}

// ---------------------------------------------------------------------------
// fp32 path (small heads/dims): one workgroup per query token, one head at a
// time; logits of all slots in LDS, two-pass softmax, then one thread per
// value column.
constexpr int NTF = 256;

__global__ __launch_bounds__(NTF) void sparse_attn_f32(
    const float* __restrict__ q, const float* __restrict__ kv, const int32_t* __restrict__ idx,
    float* __restrict__ out, float* __restrict__ lse, int T, int N, int Hn, int dqk, int dv, int k,
    float sm_scale) {
    __shared__ float z[SLOTS];
    __shared__ float qrow[256];
    __shared__ float red[NTF / 64];
    const int t = blockIdx.x, b = blockIdx.y;
    const size_t row = (size_t)b * T + t;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* kv_b = kv + (size_t)b * N * dqk;
    const int32_t* ir = idx + row * k;
    for (int h = 0; h < Hn; ++h) {
        for (int d = tid; d < dqk; d += NTF) qrow[d] = q[(row * Hn + h) * dqk + d];
        __syncthreads();
        float mx = -__builtin_inff();
        for (int i = tid; i < k; i += NTF) {
            const int id = ir[i];
            float zz = -__builtin_inff();
            if (id >= 0 && id < N) {
                const float* kr = kv_b + (size_t)id * dqk;
                float acc = 0.f;
                for (int d = 0; d < dqk; ++d) acc = fmaf(qrow[d], kr[d], acc);
                zz = acc * sm_scale;
            }
            z[i] = zz;
            mx = fmaxf(mx, zz);
        }
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        mx = red[0];
        for (int w = 1; w < NTF / 64; ++w) mx = fmaxf(mx, red[w]);
        __syncthreads();
        float sum = 0.f;
        for (int i = tid; i < k; i += NTF) {
            const float e = z[i] == -__builtin_inff() ? 0.f : expf(z[i] - mx);
            z[i] = e;
            sum += e;
        }
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
        if (lane == 0) red[wave] = sum;
        __syncthreads();
        float l = 0.f;
        for (int w = 0; w < NTF / 64; ++w) l += red[w];
        for (int v = tid; v < dv; v += NTF) {
            float acc = 0.f;
            for (int i = 0; i < k; ++i) {
                const int id = ir[i];
                if (id >= 0 && id < N) acc = fmaf(z[i], kv_b[(size_t)id * dqk + v], acc);
            }
            out[(row * Hn + h) * dv + v] = l > 0.f ? acc / l : 0.f;
        }
        if (lse != nullptr && tid == 0) lse[row * Hn + h] = l > 0.f ? mx + logf(l) : -__builtin_inff();
        __syncthreads();
    }
}

}  // namespace

int attn_num_splits(int rows, int k) {
    // enough workgroups to cover the 256 CUs; each split keeps >= 256 slots
    if (rows >= 256) return 1;
    int s = (256 + rows - 1) / rows;
    const int max_s = std::max(1, k / 256);
    return std::max(1, std::min(s, max_s));
}

size_t attn_workspace_bytes(int B, int T, int H_, int d_v, int k, dsa_dtype dtype) {
    if (dtype != DSA_BF16) return 0;
    const long long rows = (long long)B * T;
    const int s = attn_num_splits((int)std::min<long long>(rows, 1 << 30), k);
    if (s <= 1) return 0;
    return align_up((size_t)rows * s * H_ * d_v * sizeof(float)) +
           align_up((size_t)rows * s * H_ * 2 * sizeof(float));
}

dsa_status launch_attn_bf16(const void* q, const void* kv, const int32_t* idx, void* out,
                            float* lse, int B, int T, int N, int k, float sm_scale,
                            void* workspace, hipStream_t stream) {
    if (k > SLOTS) return DSA_ERR_UNSUPPORTED;
    if (T > 65535 || B > 65535) return DSA_ERR_UNSUPPORTED;
    const long long rows = (long long)B * T;
    const int s = attn_num_splits((int)std::min<long long>(rows, 1 << 30), k);
    const float scale_log2 = sm_scale * kLog2e;
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(kv);
    auto* oo = static_cast<uint16_t*>(out);
    if (s <= 1) {
        sparse_mla_attn_bf16<false><<<dim3(1, T, B), NTA, 0, stream>>>(
            qq, kk, idx, oo, lse, nullptr, nullptr, T, N, k, k, scale_log2);
        return launch_status();
    }
    const int per = ((k + s - 1) / s + TK - 1) / TK * TK;
    const int s_eff = (k + per - 1) / per;
    float* part_o = static_cast<float*>(workspace);
    float* part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              align_up((size_t)rows * s * H * DV * sizeof(float)));
    sparse_mla_attn_bf16<true><<<dim3(s_eff, T, B), NTA, 0, stream>>>(
        qq, kk, idx, oo, lse, part_o, part_ml, T, N, k, per, scale_log2);
    dsa_status st = launch_status();
    if (st != DSA_OK) return st;
    attn_combine<<<dim3((unsigned)rows), DV, 0, stream>>>(part_o, part_ml, oo, lse, s_eff);
    return launch_status();
}

dsa_status launch_attn_f32(const float* q, const float* kv, const int32_t* idx, float* out,
                           float* lse, int B, int T, int N, int Hn, int d_qk, int d_v, int k,
                           float sm_scale, hipStream_t stream) {
    if (k > SLOTS || d_qk > 256 || Hn > 32) return DSA_ERR_UNSUPPORTED;
    if (B > 65535) return DSA_ERR_UNSUPPORTED;
    sparse_attn_f32<<<dim3(T, B), NTF, 0, stream>>>(q, kv, idx, out, lse, T, N, Hn, d_qk, d_v, k,
                                                    sm_scale);
    return launch_status();
}

}  // namespace dsa
