// Sparse MLA attention backward in MQA mode on gfx950 (bf16).
//
// Method ("Paper Breakdown: DeepSeek-V3.2", section 2, "Continued
// Pre-Training (§2.1.1)": the sparse training stage trains the main model
// through the sparse attention).  With z[h,i] = scale q[h].c_i over the
// selected latent entries c_i (576 wide, shared by the 128 heads), P the
// softmax of z over the valid slots and o[h] = sum_i P[h,i] c_i[:512]:
//     dP[h,i] = do[h] . c_i[:512],   D[h] = do[h] . o[h]
//     dS[h,i] = scale P[h,i] (dP[h,i] - D[h])
//     dq[h]   = sum_i dS[h,i] c_i
//     dc_i    = sum_h dS[h,i] q[h]  (+ sum_h P[h,i] do[h] on the first 512)
// P comes back from the forward's log-sum-exp: P = exp(z - lse).
//
// Two kernels per block of query rows:
//  * sparse_mla_bwd_dq: one workgroup (4 waves, 16 heads each) per query
//    row and half of its heads.  The selected latent rows are gathered into
//    LDS 32 at a time through the same four-stage direct-to-LDS ring as the
//    forward.  Per tile and wave, S^T and dP^T (key x head) come from one
//    pass over the key fragments (the value is the key's leading 512
//    columns, so the dP^T MFMAs reuse the first 16 of the 18 key fragments);
//    P and dS are formed in fp32, rounded to bf16, written to the workspace
//    as [row][tile][head][32 slots] for the second kernel, and dS feeds
//    dq += dS C (36 MFMAs, the latent and rope columns read transposed from
//    the gathered tile).  dq (fp32) stays in AGPRs until the end.
//  * sparse_mla_bwd_dkv: one workgroup (8 waves, two per SIMD) per query
//    row.  Q and dO of the row are staged through LDS once and kept in VGPRs
//    as transposed fragments (head-major K dimension); wave w owns output
//    columns 64w..64w+63 of the latent part and waves 0..3 the rope column
//    blocks 16w..16w+15.  Per tile the
//    P and dS blocks are staged in LDS and read transposed as the A operand
//    (key x head); each slot's 576-wide vector dS^T q + P^T dO leaves the
//    kernel as one contiguous bf16 row of the workspace.
//  * the vectors are summed per token without atomics on dkv: a counting
//    sort lists the (row, slot) pairs of every token (the counts and each
//    slot's rank from sparse_mla_bwd_dq, a three-kernel exclusive scan,
//    bwd_place), then bwd_reduce gives each token one wave that adds its
//    rows in fp32 and adds the sum to dkv.
//    (fp32 atomic adds straight from sparse_mla_bwd_dkv, one per element of
//    every slot vector, took about 3.7 times as long as plain stores of the
//    same values at the chunked-prefill shape.)
#include "attn_common.h"

namespace dsa {
namespace {

constexpr int H = 128, DQK = 576, DV = 512;
constexpr int TK = 32;                    // keys per tile
constexpr int LAT = 1024;                 // latent bytes per row (512 bf16)
constexpr int ROPE = 128;                 // rope bytes per row (64 bf16)
constexpr int STAGE = TK * (LAT + ROPE);  // 36 KiB per ring stage
constexpr int SLOTS = 2048;               // max index slots of a row
constexpr int DMA_PER_TILE = 9;           // direct-to-LDS loads per wave and tile
constexpr int NT = 256;                   // threads per workgroup (4 waves)
constexpr int HG = 64;                    // heads per dq workgroup
constexpr int TILE_ELEMS = H * TK;        // one P or dS tile: [128 heads][32 slots] bf16

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// indices of one row into sidx (padded with -1 to a whole tile); returns the
// position of the last valid slot (-1 if none)
template <int NTH>
__device__ __forceinline__ int load_slots(const int32_t* __restrict__ idx_row, int k, int N,
                                          int32_t* sidx, int* s_last) {
    const int tid = threadIdx.x;
    if (tid == 0) *s_last = -1;
    __syncthreads();
    int my_last = -1;
    const int k_pad = (k + TK - 1) / TK * TK;
    // every load is issued before the first is waited for
    constexpr int PER = (SLOTS + NTH - 1) / NTH;
    int id[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + j * NTH;
        id[j] = i < k ? idx_row[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + j * NTH;
        if (i < k_pad) {
            sidx[i] = id[j];
            if (id[j] >= 0 && id[j] < N) my_last = i;
        }
    }
    if (my_last >= 0) atomicMax(s_last, my_last);
    __syncthreads();
    return *s_last;
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_bwd_dq(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const int32_t* __restrict__ idx, const uint16_t* __restrict__ out,
                       const float* __restrict__ lse, const uint16_t* __restrict__ dout,
                       float* __restrict__ dq, uint16_t* __restrict__ ws_p,
                       uint16_t* __restrict__ ws_ds, int* __restrict__ cnt, int* __restrict__ rank,
                       long long row0, int rows, int T, int N, int k, int ntile, float scale_log2,
                       float sm_scale) {
    __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st3[STAGE];
    __shared__ __attribute__((aligned(16))) int32_t sidx[SLOTS + TK];
    __shared__ __attribute__((aligned(16))) uint8_t sds[4 * 1024];  // dS fragments of the 4 waves
    __shared__ int s_last;

    // the two head halves of a row get ids 16j + x and 16j + 8 + x: the same
    // XCD (id % 8), dispatched back to back, so the second gather of the row's
    // latent rows finds them in that XCD's L2
    const unsigned id = blockIdx.x;
    const int lrow = (int)((id >> 4) * 8 + (id & 7));
    const int hg = (int)((id >> 3) & 1);
    if (lrow >= rows) return;
    const size_t row = (size_t)row0 + lrow;
    const int b = (int)(row / (unsigned)T);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, g = lane >> 4;
    const uint16_t* __restrict__ kv_b = kv + (size_t)b * N * DQK;
    const int head = hg * HG + 16 * wave + m;  // this lane's head in S^T / dP^T

    const int last = load_slots<NT>(idx + row * k, k, N, sidx, &s_last);
    const int n_tiles = (last + TK) / TK;
    const int dummy = last >= 0 ? sidx[last] : 0;

    // the per-token count of the dkv sum: the first head half's workgroup
    // counts the row's valid slots into cnt and keeps each slot's rank (the
    // atomics' latency overlaps the gather and products that follow)
    if (hg == 0) {
        const int k_pad = ntile * TK;
        constexpr int PER = (SLOTS + NT - 1) / NT;
        int rr[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NT;
            const int sid = i < k_pad ? sidx[i] : -1;
            rr[j] = (unsigned)sid < (unsigned)N ? atomicAdd(&cnt[(long long)b * N + sid], 1) : -1;
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NT;
            if (i < k_pad) rank[(size_t)lrow * k_pad + i] = rr[j];
        }
    }

    // LDS offsets inside a stage (same tile layout as the forward):
    // key fragments (chunk 4*ks + g of row m), rope fragments, and the
    // transposed reads of the latent columns (rows 4g + m/4 and +16).
    int qk_off[4];
    {
        const int sw = swz(m);
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2)
            qk_off[b2] = m * LAT + 16 * (4 * (b2 ^ (sw >> 2)) + (g ^ (sw & 3)));
    }
    int rope_off[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) rope_off[a] = TK * LAT + m * ROPE + 16 * ((4 * a + g) ^ (m & 7));
    // transposed reads (rows tr_r and tr_r + 16): latent column block cb
    // (< 32) is chunk 2*cb + (m%4)/2 of the row, in slot chunk ^ swz(row);
    // rope column block nr is rope chunk 2*nr + (m%4)/2, in slot
    // chunk ^ (row % 8)
    const int tr_r = 4 * g + (m >> 2);
    const int tr_sw = swz(tr_r);
    const int tr_base = tr_r * LAT + 16 * (((m & 3) >> 1) ^ (tr_sw & 1)) + 8 * (m & 1);
    const int tr_hi = tr_sw >> 1;
    const int trr_base = TK * LAT + tr_r * ROPE + 8 * (m & 1);
    const int trr_ch = (m & 3) >> 1, trr_sw = tr_r & 7;

    const i32x4 kv_rsrc = buffer_rsrc(kv_b, (unsigned)N * (unsigned)(2 * DQK));
    const int lane16 = lane << 4;
    auto gather_id = [&](int tile) __attribute__((always_inline)) {
        // (tiles past the last are never gathered: their loads are issued
        // with an out-of-range offset)
        const int r = 8 * wave + (lane >> 3);
        int sid = sidx[max(min(tile, n_tiles - 1), 0) * TK + r];
        if (sid < 0 || sid >= N) sid = dummy;
        return tile < n_tiles ? sid : -1;
    };
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto dma = [&](uint8_t* st, int sid, int u) __attribute__((always_inline)) {
        if (u < 8) {
            const int ru = 8 * wave_s + u;
            const int idu = __builtin_amdgcn_readlane(sid, 8 * u);
            const unsigned vo = idu < 0 ? 0x80000000u : (unsigned)(lane16 ^ (swz(ru) << 4));
            load_lds16(kv_rsrc, lds_addr(st) + ru * LAT, vo, (unsigned)max(idu, 0) * (2 * DQK));
        } else {
            const int r = 8 * wave + (lane >> 3);
            const unsigned vo = sid < 0 ? 0x80000000u
                                        : (unsigned)sid * (2 * DQK) + 1024 + 16 * ((lane & 7) ^ (r & 7));
            load_lds16(kv_rsrc, lds_addr(st) + TK * LAT + wave_s * 1024, vo, 0u);
        }
    };
    auto issue = [&](uint8_t* st, int tile) __attribute__((always_inline)) {
        const int sid = gather_id(tile);
#pragma unroll
        for (int u = 0; u < DMA_PER_TILE; ++u) dma(st, sid, u);
    };

    bf16x8 qf[DQK / 32], dof[DV / 32];
    // dq of all 64 heads (4 blocks of 16) at this wave's 9 column blocks
    // 9w..9w+8 (columns 144w..144w+143)
    const int cb0 = 9 * wave_s;
    f32x4 dqa[4][9];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int j = 0; j < 9; ++j) dqa[hb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float D = 0.f, lse2 = 0.f;

    auto compute = [&](const uint8_t* st, int tile, uint8_t* nxt) __attribute__((always_inline)) {
        const int nid = gather_id(tile + 3);
        const int4 ia = *reinterpret_cast<const int4*>(&sidx[tile * TK + 4 * g]);
        const int4 ib = *reinterpret_cast<const int4*>(&sidx[tile * TK + 16 + 4 * g]);

        // S^T and dP^T [key, head] for keys 16*nb + 4*g + i, head `head`
        f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 dacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        auto kfrag = [&](int nb, int ks) __attribute__((always_inline)) -> bf16x8 {
            const uint8_t* p = ks < 16 ? st + nb * 16 * LAT + qk_off[ks & 3] + 256 * (ks >> 2)
                                       : st + rope_off[ks - 16] + nb * 16 * ROPE;
            return as_bf16x8(*reinterpret_cast<const uint4*>(p));
        };
        bf16x8 kf[3][2];
        kf[0][0] = kfrag(0, 0); kf[0][1] = kfrag(1, 0);
        kf[1][0] = kfrag(0, 1); kf[1][1] = kfrag(1, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            const int c = ks % 3;
            if (ks + 2 < 18) {
                kf[(ks + 2) % 3][0] = kfrag(0, ks + 2);
                kf[(ks + 2) % 3][1] = kfrag(1, ks + 2);
            }
            sacc[0] = mfma_bf16(kf[c][0], qf[ks], sacc[0]);
            sacc[1] = mfma_bf16(kf[c][1], qf[ks], sacc[1]);
            if (ks < 16) {
                dacc[0] = mfma_bf16(kf[c][0], dof[ks], dacc[0]);
                dacc[1] = mfma_bf16(kf[c][1], dof[ks], dacc[1]);
            }
            if ((ks & 1) == 0) dma(nxt, nid, ks >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }

        // P = exp(z - lse) and dS = scale P (dP - D); invalid slots get 0
        const int ids[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
        float p[8], ds[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool ok = (unsigned)ids[i] < (unsigned)N;
            const float x = ok ? sacc[i >> 2][i & 3] * scale_log2 - lse2 : -__builtin_inff();
            p[i] = __builtin_amdgcn_exp2f(x);
            ds[i] = sm_scale * p[i] * (dacc[i >> 2][i & 3] - D);
        }
        const bf16x8 dsa = {(__bf16)ds[0], (__bf16)ds[1], (__bf16)ds[2], (__bf16)ds[3],
                            (__bf16)ds[4], (__bf16)ds[5], (__bf16)ds[6], (__bf16)ds[7]};
        // P^T and dS^T of this tile for the dkv kernel: head row `head`,
        // slots 4g..4g+3 and 16+4g..16+4g+3
        {
            const size_t o = ((size_t)(lrow * ntile + tile) * H + head) * TK + 4 * g;
            *reinterpret_cast<uint2*>(ws_p + o) = uint2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
            *reinterpret_cast<uint2*>(ws_p + o + 16) = uint2{pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
            *reinterpret_cast<uint2*>(ws_ds + o) = uint2{pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3])};
            *reinterpret_cast<uint2*>(ws_ds + o + 16) =
                uint2{pack_bf16(ds[4], ds[5]), pack_bf16(ds[6], ds[7])};
        }

        // dq[head, col] += dS[head, key] C[key, col].  The waves trade their
        // dS fragments through LDS, so that each multiplies all 64 heads
        // against its own nine column blocks: every C^T fragment (two
        // transposed reads: keys 4g..4g+3 and 16+4g..16+4g+3 of column
        // 16*cb + m) is read once per workgroup instead of once per wave.
        *reinterpret_cast<bf16x8*>(sds + wave * 1024 + lane * 16) = dsa;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        bf16x8 da[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) da[hb] = *reinterpret_cast<const bf16x8*>(sds + hb * 1024 + lane * 16);
        auto cfrag = [&](int cb) __attribute__((always_inline)) -> bf16x8 {
            const bool lat = cb < 32;
            const int off = lat ? tr_base + 32 * ((cb & 7) ^ tr_hi) + 256 * (cb >> 3)
                                : trr_base + 16 * ((2 * (cb - 32) + trr_ch) ^ trr_sw);
            const int step16 = lat ? 16 * LAT : 16 * ROPE;
            const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + off));
            const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + off + step16));
            const uint4 vv = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 0, 1)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 2, 3))};
            return as_bf16x8(vv);
        };
        bf16x8 cf[3];
        cf[0] = cfrag(cb0);
        cf[1] = cfrag(cb0 + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            if (j + 2 < 9) cf[(j + 2) % 3] = cfrag(cb0 + j + 2);
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) dqa[hb][j] = mfma_bf16(da[hb], cf[j % 3], dqa[hb][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto step = [&](uint8_t* cur, uint8_t* nxt, int it) __attribute__((always_inline)) {
        if (it >= n_tiles) return;
        // the stores of earlier tiles count in vmcnt too; they were issued
        // after the loads of this tile, so waiting for at most two tiles of
        // loads (plus those stores) outstanding still covers this tile
        DSA_WAIT_VM(2 * DMA_PER_TILE);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        compute(cur, it, nxt);
    };

    issue(st0, 0);
    issue(st1, 1);
    issue(st2, 2);
    {
        const uint16_t* qh = q + (row * H + head) * DQK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < DQK / 32; ++ks)
            qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qh + 32 * ks));
        const uint16_t* dh = dout + (row * H + head) * DV + 8 * g;
        const uint16_t* oh = out + (row * H + head) * DV + 8 * g;
        float d = 0.f;
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) {
            dof[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(dh + 32 * ks));
            const bf16x8 of = as_bf16x8(*reinterpret_cast<const uint4*>(oh + 32 * ks));
#pragma unroll
            for (int j = 0; j < 8; ++j) d += (float)dof[ks][j] * (float)of[j];
        }
        d += __shfl_xor(d, 16, 64);
        d += __shfl_xor(d, 32, 64);
        D = d;
        lse2 = lse[row * H + head] * kLog2e;
    }
    DSA_WAIT_VM(0);

    for (int it = 0; it < n_tiles; it += 4) {
        step(st0, st3, it);
        step(st1, st0, it + 1);
        step(st2, st1, it + 2);
        step(st3, st2, it + 3);
    }
    DSA_WAIT_VM(0);

    // dq rows 16*hb + 4g + i of the workgroup's 64 heads, column
    // 16*(cb0 + j) + m
    float* dqw = dq + (row * H + hg * HG + 4 * g) * DQK + 16 * cb0 + m;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int j = 0; j < 9; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) dqw[(16 * hb + i) * DQK + 16 * j] = dqa[hb][j][i];
}

// LDS row pitch of the staged Q and dO rows (16 bytes of padding keep the
// transposed fragment reads of four consecutive rows on different banks)
constexpr int QPITCH = 2 * DQK + 16;
constexpr int OPITCH = 2 * DV + 16;
constexpr int STAGE_B = H * QPITCH;  // 149,504 bytes
constexpr int SPITCH = 2 * DQK + 16;  // LDS pitch of a staged contribution row
// LDS pitch of a staged P or dS tile row (32 slots = 64 bytes, padded so that
// the four row groups of a transposed fragment read fall on different banks)
constexpr int TPITCH = 96;
constexpr int NTK = 512;  // threads of the dkv kernel (8 waves, 2 per SIMD)
constexpr int TILE_LDS = H * TPITCH;  // 12 KiB

__global__ __launch_bounds__(NTK) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_mla_bwd_dkv(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
                        const int32_t* __restrict__ idx, const uint16_t* __restrict__ ws_p,
                        const uint16_t* __restrict__ ws_ds, uint16_t* __restrict__ contrib,
                        long long row0, int rows, int T, int N, int k, int ntile) {
    __shared__ __attribute__((aligned(16))) uint8_t buf[STAGE_B];
    __shared__ __attribute__((aligned(16))) int32_t sidx[SLOTS + TK];
    __shared__ int s_last;

    const int lrow = blockIdx.x;
    if (lrow >= rows) return;
    const size_t row = (size_t)row0 + lrow;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, g = lane >> 4;

    const int last = load_slots<NTK>(idx + row * k, k, N, sidx, &s_last);
    const int n_tiles = (last + TK) / TK;
    if (n_tiles == 0) return;

    // transposed B fragments: heads {4g..4g+3, 16+4g..16+4g+3} + 32*kk of
    // column 16*cb + m, from rows of `pitch` bytes staged in buf
    auto tfrag = [&](int pitch, int cb, int kk) __attribute__((always_inline)) -> bf16x8 {
        const uint8_t* p = buf + (32 * kk + 4 * g + (m >> 2)) * pitch + 2 * (16 * cb + 4 * (m & 3));
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * pitch));
        const uint4 vv = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 0, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 2, 3))};
        return as_bf16x8(vv);
    };

    // this wave's column blocks: latent blocks 4w..4w+3 (value and key
    // parts) and, for waves 0..3, rope block 32 + w (key part only)
    const bool rope = wave < 4;
    auto qcb = [&](int j) __attribute__((always_inline)) { return j < 4 ? 4 * wave + j : 32 + (wave & 3); };
    bf16x8 qt[5][4], ot[4][4];
    {
        const uint16_t* qr = q + row * H * DQK;
#pragma unroll 18
        for (int it = 0; it < H * (DQK / 8) / NTK; ++it) {
            const int c = tid + it * NTK;
            const int r = c / (DQK / 8), cc = c % (DQK / 8);
            *reinterpret_cast<uint4*>(buf + r * QPITCH + 16 * cc) =
                *reinterpret_cast<const uint4*>(qr + r * DQK + 8 * cc);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 5; ++j)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qt[j][kk] = tfrag(QPITCH, qcb(j), kk);
        __syncthreads();
        const uint16_t* dr = dout + row * H * DV;
#pragma unroll 16
        for (int it = 0; it < H * (DV / 8) / NTK; ++it) {
            const int c = tid + it * NTK;
            const int r = c / (DV / 8), cc = c % (DV / 8);
            *reinterpret_cast<uint4*>(buf + r * OPITCH + 16 * cc) =
                *reinterpret_cast<const uint4*>(dr + r * DV + 8 * cc);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) ot[j][kk] = tfrag(OPITCH, 4 * wave + j, kk);
        __syncthreads();
    }

    // P and dS tiles ([128 heads][32 slots] bf16, 8 KiB each) staged in two
    // buffers, each row padded to TPITCH bytes; each thread moves 16 bytes
    // of each
    const size_t tile0 = (size_t)lrow * ntile;
    uint4 rp, rd;
    auto fetch = [&](int tile) __attribute__((always_inline)) {
        rp = reinterpret_cast<const uint4*>(ws_p + (tile0 + tile) * TILE_ELEMS)[tid];
        rd = reinterpret_cast<const uint4*>(ws_ds + (tile0 + tile) * TILE_ELEMS)[tid];
    };
    auto put = [&](int slot) __attribute__((always_inline)) {
        uint8_t* bp = buf + slot * 2 * TILE_LDS + (tid >> 2) * TPITCH + 16 * (tid & 3);
        *reinterpret_cast<uint4*>(bp) = rp;
        *reinterpret_cast<uint4*>(bp + TILE_LDS) = rd;
    };
    static_assert(NTK * 8 == TILE_ELEMS, "one 16-byte piece of each tile per thread");
    // A fragments (key x head): slots 16*kb + m, heads {4g..4g+3,
    // 16+4g..16+4g+3} + 32*kk, from a [head][32 slots] tile
    auto afrag = [&](const uint8_t* tb, int kb, int kk) __attribute__((always_inline)) -> bf16x8 {
        const uint8_t* p = tb + (32 * kk + 4 * g + (m >> 2)) * TPITCH + 2 * (16 * kb + 4 * (m & 3));
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * TPITCH));
        const uint4 vv = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 0, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 2, 3))};
        return as_bf16x8(vv);
    };

    // staged contribution rows of one tile, after the two tile buffers
    uint8_t* stg = buf + 4 * TILE_LDS;
    fetch(0);
    put(0);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        if (t + 1 < n_tiles) fetch(t + 1);
        const uint8_t* tp = buf + (t & 1) * 2 * TILE_LDS;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8 ap[4], ad[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                ad[kk] = afrag(tp + TILE_LDS, kb, kk);
                ap[kk] = afrag(tp, kb, kk);
            }
            f32x4 acc[5];
#pragma unroll
            for (int j = 0; j < 5; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = mfma_bf16(ad[kk], qt[j][kk], acc[j]);
                if (rope) acc[4] = mfma_bf16(ad[kk], qt[4][kk], acc[4]);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = mfma_bf16(ap[kk], ot[j][kk], acc[j]);
            }
            // rows of acc: slots 16*kb + 4g + i, column 16*cb + m.  Lanes m and
            // m^1 trade one value so that each writes two adjacent columns of
            // one slot row (a 32-bit LDS store) into the staged tile.
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                if (j == 4 && !rope) break;
                const int col = 16 * qcb(j) + (m & ~1);
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    const float a0 = acc[j][2 * ip], a1 = acc[j][2 * ip + 1];
                    // swap with lane m^1 (DPP quad_perm [1,0,3,2]: no LDS round trip)
                    const float recv = __int_as_float(__builtin_amdgcn_update_dpp(
                        0, __float_as_int((m & 1) ? a0 : a1), 0xB1, 0xF, 0xF, false));
                    const int r = 16 * kb + 4 * g + 2 * ip + (m & 1);
                    *reinterpret_cast<uint32_t*>(stg + r * SPITCH + 2 * col) =
                        (m & 1) ? pack_bf16(recv, a1) : pack_bf16(a0, recv);
                }
            }
        }
        // the tile's 32 contribution rows (576 bf16 each) to the workspace
        __syncthreads();
        uint16_t* dst = contrib + ((size_t)lrow * (ntile * TK) + t * TK) * DQK;
#pragma unroll
        for (int it = 0; it < (TK * (DQK / 8) + NTK - 1) / NTK; ++it) {
            const int c = tid + it * NTK;
            if (c < TK * (DQK / 8)) {
                const int r = c / (DQK / 8), cc = c % (DQK / 8);
                *reinterpret_cast<uint4*>(dst + r * DQK + 8 * cc) =
                    *reinterpret_cast<const uint4*>(stg + r * SPITCH + 16 * cc);
            }
        }
        if (t + 1 < n_tiles) put((t + 1) & 1);
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void zero_f32(float4* __restrict__ p, size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        p[i] = float4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(256) void zero_i32(int* __restrict__ p, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// ---------------------------------------------------------------------------
// Sum of the contribution rows per token.  A pair p = lrow * k_pad + slot of
// the block's rows selects token key = b * N + idx; the pairs of each token
// are listed contiguously (counting sort: the counts with ranks, taken by
// sparse_mla_bwd_dq, an exclusive scan of the counts, placement), then one
// wave per token adds its rows.  When the
// batch has many more cache rows than a block has pairs (decode-shaped
// batches), placement also lists the tokens that have pairs (the pair of rank
// 0 appends its token; cnt[nkeys] counts them), so the sum runs over the
// selected tokens only, not over every row of the cache.

constexpr int SCAN_CHUNK = 2048;  // counts per scan workgroup (256 threads x 8)

// inclusive scan of one value per thread over a 256-thread workgroup
__device__ __forceinline__ int block_scan256(int v, int* s_w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_w[wave] = v;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += s_w[w];
    __syncthreads();
    return v + add;
}

__global__ __launch_bounds__(256) void scan_chunk_sums(const int* __restrict__ cnt, int* __restrict__ sums,
                                                      long long n) {
    __shared__ int s_w[4];
    const long long base = (long long)blockIdx.x * SCAN_CHUNK + threadIdx.x * 8;
    int v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (base + j < n) v += cnt[base + j];
    v = block_scan256(v, s_w);
    if (threadIdx.x == 255) sums[blockIdx.x] = v;
}

// exclusive scan of the chunk sums in place (one workgroup)
__global__ __launch_bounds__(256) void scan_sums(int* __restrict__ sums, int nchunks) {
    __shared__ int s_w[4];
    __shared__ int s_carry;
    if (threadIdx.x == 0) s_carry = 0;
    __syncthreads();
    for (int b0 = 0; b0 < nchunks; b0 += 256) {
        const int i = b0 + threadIdx.x;
        const int v = i < nchunks ? sums[i] : 0;
        const int inc = block_scan256(v, s_w);
        const int carry = s_carry;
        if (i < nchunks) sums[i] = carry + inc - v;
        __syncthreads();
        if (threadIdx.x == 255) s_carry = carry + inc;
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void scan_apply(const int* __restrict__ cnt, const int* __restrict__ sums,
                                                 int* __restrict__ off, long long n) {
    __shared__ int s_w[4];
    const long long base = (long long)blockIdx.x * SCAN_CHUNK + threadIdx.x * 8;
    int c[8], v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        c[j] = base + j < n ? cnt[base + j] : 0;
        v += c[j];
    }
    int run = block_scan256(v, s_w) - v + sums[blockIdx.x];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (base + j < n) off[base + j] = run;
        run += c[j];
    }
}

__global__ __launch_bounds__(256) void bwd_place(const int32_t* __restrict__ idx, const int* __restrict__ off,
                                                const int* __restrict__ rank, int* __restrict__ list,
                                                int* __restrict__ cnt, int* __restrict__ touched,
                                                long long nkeys, long long row0, int rows, int T, int N,
                                                int k, int k_pad) {
    __shared__ int s_n, s_base;
    const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
    const int r = p < (long long)rows * k_pad ? rank[p] : -1;
    long long key = 0;
    if (r >= 0) {
        const int lrow = (int)(p / k_pad), slot = (int)(p % k_pad);
        const long long row = row0 + lrow;
        const int id = idx[row * k + slot];
        key = (row / T) * N + id;
        list[off[key] + r] = (int)p;
    }
    if (!touched) return;
    // the workgroup's first pairs append their tokens with one global atomic
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    const int loc = r == 0 ? atomicAdd(&s_n, 1) : 0;
    __syncthreads();
    if (threadIdx.x == 0 && s_n > 0) s_base = atomicAdd(&cnt[nkeys], s_n);
    __syncthreads();
    if (r == 0) touched[s_base + loc] = (int)key;
}

__device__ __forceinline__ void add_bf16x8(float* a, const uint4& x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[2 * j] += __uint_as_float(w[j] << 16);
        a[2 * j + 1] += __uint_as_float(w[j] & 0xffff0000u);
    }
}

// one wave per token (touched == NULL) or per listed token: lane l adds
// 16-byte chunks l and (l < 8) l + 64 of the token's contribution rows (72
// chunks of 8 bf16), four rows per round, then adds the sum to dkv (earlier
// blocks' sums are already there)
__global__ __launch_bounds__(256) void bwd_reduce(const uint16_t* __restrict__ contrib,
                                                 const int* __restrict__ cnt, const int* __restrict__ off,
                                                 const int* __restrict__ list, const int* __restrict__ touched,
                                                 float* __restrict__ dkv, long long nkeys, int overwrite) {
    const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= (touched ? (long long)cnt[nkeys] : nkeys)) return;
    const long long key = touched ? (long long)touched[w] : w;
    const int n = cnt[key];
    const int lane = threadIdx.x & 63;
    if (n == 0) {
        // (overwrite: the first block of a call that visits every cache row
        // writes the whole of dkv, zeros for the rows without pairs)
        if (overwrite) {
            float4* d = reinterpret_cast<float4*>(dkv + key * DQK);
            for (int c = lane; c < DQK / 4; c += 64) d[c] = float4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }
    const bool two = lane < DQK / 8 - 64;
    const int o = off[key];
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int e0 = 0; e0 < n; e0 += 64) {
        const int ne = min(64, n - e0);
        const int pv = lane < ne ? list[o + e0 + lane] : 0;
        for (int e = 0; e < ne; e += 4) {
            uint4 xa[4], xb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pu = __shfl(pv, min(e + u, ne - 1), 64);
                const uint16_t* src = contrib + (size_t)pu * DQK;
                xa[u] = e + u < ne ? *reinterpret_cast<const uint4*>(src + 8 * lane) : uint4{0u, 0u, 0u, 0u};
                xb[u] = (two && e + u < ne) ? *reinterpret_cast<const uint4*>(src + 8 * (lane + 64))
                                            : uint4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                add_bf16x8(a, xa[u]);
                add_bf16x8(b, xb[u]);
            }
        }
    }
    float4* d = reinterpret_cast<float4*>(dkv + key * DQK);
    const float4 zero = {0.f, 0.f, 0.f, 0.f};
    float4 d0 = overwrite ? zero : d[2 * lane], d1 = overwrite ? zero : d[2 * lane + 1];
    d[2 * lane] = float4{d0.x + a[0], d0.y + a[1], d0.z + a[2], d0.w + a[3]};
    d[2 * lane + 1] = float4{d1.x + a[4], d1.y + a[5], d1.z + a[6], d1.w + a[7]};
    if (two) {
        float4 e0v = overwrite ? zero : d[2 * (lane + 64)], e1v = overwrite ? zero : d[2 * (lane + 64) + 1];
        d[2 * (lane + 64)] = float4{e0v.x + b[0], e0v.y + b[1], e0v.z + b[2], e0v.w + b[3]};
        d[2 * (lane + 64) + 1] = float4{e1v.x + b[4], e1v.y + b[5], e1v.z + b[6], e1v.w + b[7]};
    }
}

// rows per block of the kernels (the workspace holds one block's P and dS
// tiles, contribution rows and lists)
constexpr long long kBwdRows = 2048;

struct BwdLayout {
    size_t p, ds, contrib, rank, list, cnt, off, sums, touched, total;
};

BwdLayout bwd_layout(long long rows, long long nkeys, int k) {
    const long long rb = rows < kBwdRows ? rows : kBwdRows;
    const size_t ntile = (size_t)(k + TK - 1) / TK;
    const size_t pairs = (size_t)rb * ntile * TK;
    BwdLayout L;
    size_t at = 0;
    auto take = [&](size_t bytes) { const size_t a = at; at += align_up(bytes); return a; };
    L.p = take((size_t)rb * ntile * TILE_ELEMS * sizeof(uint16_t));
    L.ds = take((size_t)rb * ntile * TILE_ELEMS * sizeof(uint16_t));
    L.contrib = take(pairs * DQK * sizeof(uint16_t));
    L.rank = take(pairs * sizeof(int));
    L.list = take(pairs * sizeof(int));
    L.cnt = take((size_t)(nkeys + 1) * sizeof(int));  // + the count of listed tokens
    L.off = take((size_t)nkeys * sizeof(int));
    L.sums = take((size_t)((nkeys + SCAN_CHUNK - 1) / SCAN_CHUNK) * sizeof(int));
    L.touched = take((size_t)std::min<long long>(nkeys, (long long)pairs) * sizeof(int));  // listed tokens
    L.total = at;
    return L;
}

}  // namespace

size_t attn_bwd_workspace_bytes(int B, int T, int N, int k) {
    return bwd_layout((long long)B * T, (long long)B * N, k).total;
}

dsa_status launch_attn_bwd_bf16(const void* q, const void* kv, const int32_t* idx, const void* out,
                                const float* lse, const void* dout, float* dq, float* dkv, int B,
                                int T, int N, int k, float sm_scale, void* workspace,
                                hipStream_t stream) {
    if (k > SLOTS) return DSA_ERR_UNSUPPORTED;
    if ((size_t)N * (2 * DQK) >= 0x80000000ull) return DSA_ERR_UNSUPPORTED;
    const long long rows = (long long)B * T, nkeys = (long long)B * N;
    const int ntile = (k + TK - 1) / TK, k_pad = ntile * TK;
    const long long rb = rows < kBwdRows ? rows : kBwdRows;
    const BwdLayout L = bwd_layout(rows, nkeys, k);
    char* w = static_cast<char*>(workspace);
    uint16_t* ws_p = reinterpret_cast<uint16_t*>(w + L.p);
    uint16_t* ws_ds = reinterpret_cast<uint16_t*>(w + L.ds);
    uint16_t* contrib = reinterpret_cast<uint16_t*>(w + L.contrib);
    int* rank = reinterpret_cast<int*>(w + L.rank);
    int* list = reinterpret_cast<int*>(w + L.list);
    int* cnt = reinterpret_cast<int*>(w + L.cnt);
    int* off = reinterpret_cast<int*>(w + L.off);
    int* sums = reinterpret_cast<int*>(w + L.sums);
    int* touched = reinterpret_cast<int*>(w + L.touched);
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(kv);
    const auto* oo = static_cast<const uint16_t*>(out);
    const auto* dd = static_cast<const uint16_t*>(dout);
    const unsigned nchunks = (unsigned)((nkeys + SCAN_CHUNK - 1) / SCAN_CHUNK);

    // dkv starts at zero: cleared here when the first block sums over a
    // list of tokens, otherwise written whole by the first block's sum
    const bool first_list = nkeys > 4 * (long long)rb * k_pad;
    dsa_status st = DSA_OK;
    if (first_list) {
        const size_t n4 = (size_t)nkeys * DQK / 4;
        DSA_TIMED("zero_f32", stream,
                  zero_f32<<<dim3((unsigned)std::min<size_t>((n4 + 255) / 256, 8192)), 256, 0, stream>>>(
                      reinterpret_cast<float4*>(dkv), n4));
        st = launch_status();
        if (st != DSA_OK) return st;
    }
    for (long long r0 = 0; r0 < rows; r0 += rb) {
        const int nr = (int)std::min<long long>(rb, rows - r0);
        const long long npairs = (long long)nr * k_pad;
        const unsigned gp = (unsigned)((npairs + 255) / 256);
        const bool use_list = nkeys > 4 * npairs;  // most cache rows unselected
        const int overwrite = r0 == 0 && !use_list ? 1 : 0;
        DSA_TIMED("zero_i32", stream,
                  zero_i32<<<dim3((unsigned)std::min<long long>((nkeys + 256) / 256, 8192)), 256, 0,
                             stream>>>(cnt, (size_t)nkeys + 1));
        DSA_TIMED("sparse_mla_bwd_dq", stream,
                  sparse_mla_bwd_dq<<<dim3((unsigned)((nr + 7) / 8 * 16)), NT, 0, stream>>>(
                      qq, kk, idx, oo, lse, dd, dq, ws_p, ws_ds, cnt, rank, r0, nr, T, N, k, ntile,
                      sm_scale * kLog2e, sm_scale));
        DSA_TIMED("sparse_mla_bwd_dkv", stream,
                  sparse_mla_bwd_dkv<<<dim3((unsigned)nr), NTK, 0, stream>>>(
                      qq, dd, idx, ws_p, ws_ds, contrib, r0, nr, T, N, k, ntile));
        DSA_TIMED("scan_chunk_sums", stream,
                  scan_chunk_sums<<<dim3(nchunks), 256, 0, stream>>>(cnt, sums, nkeys));
        DSA_TIMED("scan_sums", stream, scan_sums<<<dim3(1), 256, 0, stream>>>(sums, (int)nchunks));
        DSA_TIMED("scan_apply", stream,
                  scan_apply<<<dim3(nchunks), 256, 0, stream>>>(cnt, sums, off, nkeys));
        DSA_TIMED("bwd_place", stream,
                  bwd_place<<<dim3(gp), 256, 0, stream>>>(idx, off, rank, list, cnt,
                                                          use_list ? touched : nullptr, nkeys, r0, nr,
                                                          T, N, k, k_pad));
        // one wave per cache row, or per listed token (at most npairs of them)
        const long long nred = use_list ? npairs : nkeys;
        DSA_TIMED("bwd_reduce", stream,
                  bwd_reduce<<<dim3((unsigned)((nred + 3) / 4)), 256, 0, stream>>>(
                      contrib, cnt, off, list, use_list ? touched : nullptr, dkv, nkeys, overwrite));
        st = launch_status();
        if (st != DSA_OK) return st;
    }
    return DSA_OK;
}

}  // namespace dsa
