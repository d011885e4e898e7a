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
//    out[token, col] = c[token, :512] . W[col, :] for the 256 output
//    columns (128 key + 128 value) of one head and 256 tokens per workgroup.
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

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---------------------------------------------------------------------------
// Up-projection: out[row, col] = c[row, :512] . W[col, :] for the 256 output
// columns of one head (W_UK[h]'s 128 rows, then W_UV[h]'s) and 256 latent rows
// per workgroup (8 waves: wave w takes rows 64 (w / 2) .. +63 and the key
// (w even) or value (w odd) columns; 2 x 4 blocks of 32 x 32 fp32 per wave).
// The contraction runs in 16 chunks of 32 k: each chunk's 256 latent rows
// and 256 weight rows (64 bytes each) are staged in LDS, double-buffered,
// and its global loads are issued two chunks ahead of its product (two
// register sets), so two chunks' MFMA work covers their latency; one
// workgroup (two waves per SIMD) per CU.  A row's four 16-byte pieces
// sit at slot q ^ ((r / 4) % 4), so the 16 lanes that read one piece of 16
// consecutive rows hit distinct banks.
// bf16 v_mfma_f32_32x32x16: A = 16 bytes of a latent row, B = 16 bytes of a
// weight row (both k-contiguous).  Results go out in bf16 straight from the
// accumulators through LDS (adjacent lanes pairing columns by DPP) and out as
// 16-byte streaming stores (the 8 GiB of per-head rows would only evict the
// latent rows and weights from the caches).
// Workgroup order: workgroups are handed to the 8 XCDs in turn, so XCD x
// takes row blocks x, x + 8, ...; along one XCD the head runs fastest within
// a group of UP_HG heads, so the workgroups resident on an XCD at once share
// latent row blocks through its L2 while the group's weights stay there too.
constexpr int UP_ROWS = 256;          // latent rows per workgroup
constexpr int UP_NT = 512;            // threads per workgroup (8 waves)
constexpr int UP_HG = 8;              // heads per group (grid y = H / UP_HG)
static_assert(H % UP_HG == 0, "head groups must tile the heads");
constexpr int UP_COLS = 2 * DN;       // output columns per workgroup (one head: key + value)
constexpr int UP_BK = 32;             // k per chunk
constexpr int UP_A = UP_ROWS * UP_BK; // bf16 per A chunk
constexpr int UP_B = UP_COLS * UP_BK; // bf16 per B chunk
constexpr int UP_OPITCH = 2 * 128 + 16; // LDS bytes per staged output row (128 bf16 + pad)
constexpr int UP_LDS = 2 * (2 * UP_A + 2 * UP_B) > (UP_NT / 64) * 32 * UP_OPITCH
                           ? 2 * (2 * UP_A + 2 * UP_B) : (UP_NT / 64) * 32 * UP_OPITCH;  // bytes

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBuf = 0x00020000;  // buffer resource word 3: raw (untyped) 32-bit data

__device__ __forceinline__ int up_slot(int r, int q) { return 4 * r + (q ^ ((r >> 2) & 3)); }

__global__ __launch_bounds__(UP_NT) void mha_up_project(const uint16_t* __restrict__ kv,
                                                      const uint16_t* __restrict__ w_uk,
                                                      const uint16_t* __restrict__ w_uv,
                                                      uint16_t* __restrict__ kh,
                                                      uint16_t* __restrict__ vh, long long rows) {
    // the chunk buffers (A: 2 x UP_A, then B: 2 x UP_B); after the
    // contraction the same bytes stage the output rows
    __shared__ __attribute__((aligned(16))) uint16_t lds_ab[UP_LDS / 2];
    uint16_t* const lds_a[2] = {lds_ab, lds_ab + UP_A};
    uint16_t* const lds_b[2] = {lds_ab + 2 * UP_A, lds_ab + 2 * UP_A + UP_B};
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int s_x = blockIdx.x >> 3;  // position along XCD blockIdx.x % 8
    const int h = blockIdx.y * UP_HG + s_x % UP_HG;
    const long long r0 = ((long long)(s_x / UP_HG) * 8 + (blockIdx.x & 7)) * UP_ROWS;
    if (r0 >= rows) return;
    const int wr = wave >> 1, wc = wave & 1;  // row quarter, key / value columns
    const int i32 = lane & 31, half = lane >> 5;

    // chunk loads through buffer resources: A = 256 latent rows x 4 pieces
    // (2 per thread), B = 256 weight rows x 4 pieces (2 per thread: W_UK[h]'s
    // row, then W_UV[h]'s); thread tid moves piece tid % 4 of rows tid / 4 +
    // 128 j.  Latent rows past the end read as zeros (every offset sits in the
    // range-checked vector offset).
    const int nrow = (int)(rows - r0 < UP_ROWS ? rows - r0 : UP_ROWS);
    const auto a_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kv + (size_t)r0 * LAT_ROW), 0,
                                                        nrow * LAT_ROW * 2, kRawBuf);
    const auto k_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w_uk + (size_t)h * DN * DC), 0,
                                                        DN * DC * 2, kRawBuf);
    const auto v_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w_uv + (size_t)h * DVH * DC), 0,
                                                        DVH * DC * 2, kRawBuf);
    const int pr = tid >> 2, pq = tid & 3;
    const int a_voff = pr * LAT_ROW * 2 + 16 * pq;
    const int b_voff = pr * DC * 2 + 16 * pq;
    const int st_el = 8 * up_slot(pr, pq);  // + 128 rows = + 8192 bytes (the slot swizzle repeats)
    struct Chunk { u32x4 a[2], b[2]; };
    auto load = [&](Chunk& c, int kc) __attribute__((always_inline)) {
        const int ko = UP_BK * 2 * kc;
        c.a[0] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_voff + ko, 0, 0);
        c.a[1] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_voff + 128 * LAT_ROW * 2 + ko, 0, 0);
        c.b[0] = __builtin_amdgcn_raw_buffer_load_b128(k_rs, b_voff + ko, 0, 0);
        c.b[1] = __builtin_amdgcn_raw_buffer_load_b128(v_rs, b_voff + ko, 0, 0);
    };
    auto stage = [&](const Chunk& c, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&lds_a[buf][st_el + 4096 * j]) = c.a[j];
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&lds_b[buf][st_el + 4096 * j]) = c.b[j];
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb2][cb][e] = 0.f;

    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < UP_BK / 16; ++ks) {
            // k step ks: piece 2 ks + half of each row
            bf16x8_t af[2], bf[4];
#pragma unroll
            for (int rb2 = 0; rb2 < 2; ++rb2)
                af[rb2] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                    &lds_a[buf][8 * up_slot(64 * wr + 32 * rb2 + i32, 2 * ks + half)]));
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                bf[cb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                    &lds_b[buf][8 * up_slot(128 * wc + 32 * cb + i32, 2 * ks + half)]));
#pragma unroll
            for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[rb2][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb2], bf[cb], acc[rb2][cb], 0, 0, 0);
        }
    };

    // Chunk kc is multiplied from LDS buffer kc % 2; chunk kc + 1 waits in
    // register set (kc + 1) % 2 and chunk kc + 2 in set kc % 2, so a chunk's
    // loads have two chunks' products to land.  After chunk kc's product,
    // chunk kc + 1 goes to LDS buffer (kc + 1) % 2 (last read by chunk kc - 1,
    // before the previous barrier) and its register set takes chunk kc + 3.
    constexpr int NKC = DC / UP_BK;
    static_assert(NKC % 2 == 0 && NKC >= 4, "chunk pipeline assumes an even chunk count");
    // (scheduling barriers keep the loads where they are written: the
    // compiler would otherwise sink them next to their first use)
    Chunk c0, c1;
    load(c0, 0);
    load(c1, 1);
    stage(c0, 0);
    load(c0, 2);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < NKC; kc += 2) {
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        stage(c1, 1);
        __syncthreads();
        if (kc + 3 < NKC) load(c1, kc + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        __builtin_amdgcn_sched_barrier(0);
        if (kc + 2 < NKC) {
            stage(c0, 0);
            __syncthreads();
            if (kc + 4 < NKC) load(c0, kc + 4);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // acc[rb2][cb] register e of lane (i32, half): row 64 wr + 32 rb2 + 8 (e / 4)
    // + 4 half + e % 4, column 32 cb + i32 of the wave's 128.  Adjacent lanes
    // (i32 even / odd) trade one value so that the even lane holds columns
    // i32, i32 + 1 of row e and the odd lane columns i32 - 1, i32 of row e + 1.
    // Each half of the wave's rows (32 rows x 128 columns, bf16) is staged in
    // the wave's own LDS region and leaves as 16-byte pieces: lane l takes
    // piece l % 16 of row 4 j + l / 16, so 16 lanes write one 256-byte row
    // segment.
    const bool odd = (i32 & 1) != 0;
    uint16_t* const base = wc == 0 ? kh : vh;
    uint8_t* const stg = reinterpret_cast<uint8_t*>(lds_ab) + wave * (32 * UP_OPITCH);
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2) {
        __syncthreads();  // (the chunk buffers, then the previous half, are read)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float x0 = acc[rb2][cb][e], x1 = acc[rb2][cb][e + 1];
                const float send = odd ? x0 : x1;
                const float recv = __builtin_bit_cast(
                    float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xf, 0xf, false));
                const float lo = odd ? recv : x0, hi = odd ? x1 : recv;
                const int rl = 8 * (e >> 2) + 4 * half + (e & 3) + (odd ? 1 : 0);
                const uint32_t pk = (uint32_t)bf16_bits(lo) | ((uint32_t)bf16_bits(hi) << 16);
                *reinterpret_cast<uint32_t*>(stg + rl * UP_OPITCH + 2 * (32 * cb + (i32 & ~1))) = pk;
            }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int rl = 4 * j + (lane >> 4);
            const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rl * UP_OPITCH + 16 * (lane & 15));
            const long long gr = r0 + 64 * wr + 32 * rb2 + rl;
            if (gr < rows)
                __builtin_nontemporal_store(
                    v, reinterpret_cast<u32x4*>(base + ((size_t)gr * H + h) * DN + 8 * (lane & 15)));
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
    // up-projection grid: x = 8 XCDs x (row blocks per XCD) x UP_HG heads,
    // UP_NT threads each; the x extent in threads must stay below 2^32
    const long long up_jb = ((rows_kv + UP_ROWS - 1) / UP_ROWS + 7) / 8;
    if (rows_q > 0x7fffffffLL || up_jb * 8 * UP_HG * UP_NT > 0xffffffffLL) return DSA_ERR_UNSUPPORTED;
    auto* kh = static_cast<uint16_t*>(workspace);
    auto* vh = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                           align_up((size_t)rows_kv * H * DN * sizeof(uint16_t)));
    DSA_TIMED("mha_up_project", stream,
              mha_up_project<<<dim3((unsigned)(up_jb * 8 * UP_HG), H / UP_HG), UP_NT, 0,
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
