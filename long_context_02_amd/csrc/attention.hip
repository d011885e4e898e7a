// Sparse MLA attention in MQA mode on gfx950.
//
// Method ("Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture: DSA
// (§2.1)"): u_t = Attn(h_t, {c_s : I[t,s] in Top-k(I[t,:])}); under "DSA
// under MLA (MQA Mode)" one latent vector c_s (576 wide: 512 latent + 64
// rope) per selected token is shared by all 128 query heads, and the value
// is its 512-wide latent part.
//
// bf16 path: one workgroup (4 waves, 32 heads each, one wave per SIMD) per
// query token and slot range.  The selected latent rows are gathered 32 at a
// time (a tile) straight into LDS with direct-to-LDS loads (global_load_lds;
// no registers in flight) through a ring of four 36 KiB stages; the loads of
// tile i+3 are issued between the key-product MFMAs of tile i.  Latent rows
// are stored with their 16-byte chunks swizzled so that both the key-product
// fragment reads and the transposed value reads are free of bank conflicts.
//
// Per wave and tile:
//   S^T[key, head] = K[key, :] . Q[head, :]        18 x 4 bf16 MFMA 16x16x32
//     (A = key rows from LDS, B = the wave's 32 query heads kept in VGPRs;
//      S^T puts one head per lane column, the layout the P operand of the
//      value product needs)
//   softmax in base 2 against a fixed reference max per head (the max of
//     the first tile with a valid key): exp2(x - m_ref) may grow to
//     2^REF_GAP, which fp32 sums and bf16 weights carry without loss of
//     relative precision, so the accumulator is never rescaled; a tile that
//     exceeds the reference by more than REF_GAP makes the workgroup redo
//     the pass against the exact max it recorded
//   O[head, v] += P[head, key] V[key, v]           2 x 32 bf16 MFMA 16x16x32
//     (V^T fragments come from the latent rows in LDS through ds_read_b64_tr_b16
//      transposed reads; the key order of the MFMA's K dimension matches the
//      accumulator layout of S^T)
// The O accumulator (32 heads x 512 fp32 per wave) lives in AGPRs.  Batches
// with fewer rows than CUs split the slots over several workgroups; each
// writes its O rows normalised in bf16 with its per-head (max, exp-sum), and
// attn_combine merges them.
#include "attn_common.h"

namespace dsa {
namespace {

constexpr int H = 128, DQK = 576, DV = 512;
constexpr int NWV = 4;                   // waves per workgroup, 32 heads each
constexpr int NTA = NWV * 64;            // 256 threads
constexpr int TK = 32;                   // keys per tile
constexpr int LAT = 1024;                // latent bytes per row (512 bf16)
constexpr int ROPE = 128;                // rope bytes per row (64 bf16)
constexpr int STAGE = TK * (LAT + ROPE); // 36 KiB per ring stage
constexpr int SLOTS = 2048;              // max index slots per workgroup
constexpr float REF_GAP = 64.0f;         // max log2 gap above the reference max
constexpr int DMA_PER_TILE = 9;          // direct-to-LDS loads per wave and tile

template <bool PARTIAL>
__global__ __launch_bounds__(NTA) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml, int T, int N, int k, int nsplit, int slots_per_split,
    float scale_log2) {
    // four ring stages, separate objects so that the compiler can tell the
    // stage being read from the stages being filled
    __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st3[STAGE];
    __shared__ __attribute__((aligned(16))) int32_t sidx[SLOTS + 3 * TK];
    __shared__ int s_last;
    __shared__ int s_redo;

    // (split batches only: causal prefill rows differ in length, and giving
    // each XCD a contiguous range of them would unbalance the XCDs)
    const unsigned item = PARTIAL ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const int split = (int)(item % (unsigned)nsplit);
    const size_t row = item / (unsigned)nsplit;
    const int b = (int)(row / (unsigned)T);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, g = lane >> 4;
    const int slot0 = split * slots_per_split;
    const int nslots = max(0, min(k - slot0, slots_per_split));
    const uint16_t* __restrict__ kv_b = kv + (size_t)b * N * DQK;

    // ---- slot indices of this workgroup; the last valid one
    if (tid == 0) s_last = -1;
    __syncthreads();
    int my_last = -1;
    const int nslots_pad = (nslots + TK - 1) / TK * TK;
    // this wave's 32 query heads (two blocks of 16) as B operands
    bf16x8 qf[2][DQK / 32];
    {
        // all of a thread's index loads are issued before the first is
        // waited for (a loop that stores each index as it arrives waits for
        // one memory round trip per iteration), and Q's loads right behind
        // them, so that Q arrives while the indices are used
        constexpr int PER = (SLOTS + 3 * TK + NTA - 1) / NTA;
        int id[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTA;
            id[j] = i < nslots ? idx[row * k + slot0 + i] : -1;
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const uint16_t* qh = q + (row * H + 32 * wave + 16 * hb + m) * DQK + 8 * g;
#pragma unroll
            for (int ks = 0; ks < DQK / 32; ++ks)
                qf[hb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qh + 32 * ks));
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTA;
            if (i < nslots_pad + 3 * TK) {
                sidx[i] = id[j];
                if (id[j] >= 0 && id[j] < N) my_last = i;
            }
        }
    }
    if (my_last >= 0) atomicMax(&s_last, my_last);

    __syncthreads();
    const int last = s_last;
    const int n_tiles = (last + TK) / TK;  // 0 when no slot is valid
    // rows of invalid slots are loaded from a selected row (their weight is 0)
    const int dummy = last >= 0 ? sidx[last] : 0;

    // Softmax without rescaling the accumulator: the reference max m_ref of
    // head 16*hb + m is the max of the first tile with a valid key, and
    // later exponentials exp2(x - m_ref) may grow up to 2^REF_GAP, which fp32
    // accumulators and bf16 weights hold without loss of relative precision.
    // A tile that exceeds the reference by more than REF_GAP flags the
    // workgroup, which then reruns the pass with m_ref = the exact max it
    // recorded (so every exponential is <= 1).
    f32x4 o[2][DV / 16];
    float m_ref[2], m_all[2], l_part[2];
    bool over = false;
    if (tid == 0) s_redo = 0;

    // per-lane LDS offsets inside a stage (all rows use the same swizzle of
    // their low four bits, so these hold for every tile).  QK^T: chunk
    // 4*ks + g of row r sits in slot 4*(ks ^ (swz>>2)) + (g ^ (swz&3)).
    int qk_off[4];
    {
        const int sw = swz(m);
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2)
            qk_off[b2] = m * LAT + 16 * (4 * (b2 ^ (sw >> 2)) + (g ^ (sw & 3)));
    }
    // rope chunk 4*a + g (a = 0, 1) of row r sits in slot (4*a + g) ^ (r % 8)
    int rope_off[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) rope_off[a] = TK * LAT + m * ROPE + 16 * ((4 * a + g) ^ (m & 7));
    // P V: the K order of the MFMA is {4g..4g+3, 16+4g..16+4g+3} on both
    // operands.  V comes from the latent rows by transposed reads: lane m of
    // group g reads 8 bytes of row r = 4g + m/4 (and r + 16) at columns
    // 16*nv + 4*(m%4), i.e. chunk 2*nv + (m%4)/2, and receives column
    // 16*nv + m of those four rows.  Slot (2*nv + ch) ^ swz(r) splits into
    // 32*((nv%8) ^ (swz>>1)) + 16*(ch ^ (swz&1)) + 256*(nv/8).
    // (row r + 16 has the same swizzle, 16 KiB further on)
    int tr_off[8];
    {
        const int r = 4 * g + (m >> 2);
        const int sw = swz(r), ch = (m & 3) >> 1;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            tr_off[j] = r * LAT + 32 * (j ^ (sw >> 1)) + 16 * (ch ^ (sw & 1)) + 8 * (m & 1);
    }

    // direct-to-LDS gather of one tile: wave w brings latent rows 8w..8w+7
    // (one 1 KiB row per instruction, lane l fetching chunk l ^ swz(r)) and
    // the rope parts of rows 8w..8w+7 (lane l: row 8w+l/8, chunk
    // (l%8) ^ (row%8)); 9 loads per wave and tile.  The loads go through a
    // buffer resource over this sequence's rows (the base stays in SGPRs;
    // the row offset of a latent load is a scalar).  A tile at or past
    // n_tiles is still "loaded", with offsets beyond the resource's range:
    // such loads touch no memory, so every tile issues the same number of
    // loads and the ring's wait counts do not depend on the position.
    // gather_id() looks the rows up (lane l: row 8w + l/8); dma(u) issues
    // load u.
    const i32x4 kv_rsrc = buffer_rsrc(kv_b, (unsigned)N * (unsigned)(2 * DQK));
    const int lane16 = lane << 4;
    auto gather_id = [&](int tile) __attribute__((always_inline)) {
        // (the lookahead reaches three tiles past the last one: sidx holds
        // -1 there, and such tiles are never gathered)
        const int r = 8 * wave + (lane >> 3);
        int id = sidx[tile * TK + r];
        if (id < 0 || id >= N) id = dummy;
        return tile < n_tiles ? id : -1;
    };
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto dma = [&](uint8_t* st, int id, int u) __attribute__((always_inline)) {
        if (u < 8) {
            const int ru = 8 * wave_s + u;
            const int idu = __builtin_amdgcn_readlane(id, 8 * u);
            const unsigned vo = idu < 0 ? 0x80000000u : (unsigned)(lane16 ^ (swz(ru) << 4));
            load_lds16(kv_rsrc, lds_addr(st) + ru * LAT, vo, (unsigned)max(idu, 0) * (2 * DQK));
        } else {
            const int r = 8 * wave + (lane >> 3);
            const unsigned vo = id < 0 ? 0x80000000u
                                       : (unsigned)id * (2 * DQK) + 1024 + 16 * ((lane & 7) ^ (r & 7));
            load_lds16(kv_rsrc, lds_addr(st) + TK * LAT + wave_s * 1024, vo, 0u);
        }
    };
    auto issue = [&](uint8_t* st, int tile) __attribute__((always_inline)) {
        const int id = gather_id(tile);
#pragma unroll
        for (int u = 0; u < DMA_PER_TILE; ++u) dma(st, id, u);
    };

    // Multiply tile `tile` (in stage st); when nxt is not null, the loads of
    // tile `tile + 3` into nxt are spread over the QK^T steps.
    auto compute = [&](const uint8_t* st, int tile, uint8_t* nxt) __attribute__((always_inline)) {
        const int nid = gather_id(tile + 3);
        // validity of this lane's keys 4g..4g+3 and 16+4g..16+4g+3
        const int4 ia = *reinterpret_cast<const int4*>(&sidx[tile * TK + 4 * g]);
        const int4 ib = *reinterpret_cast<const int4*>(&sidx[tile * TK + 16 + 4 * g]);

        // S^T[key, head] for keys 16*nb + 4*g + i, heads 16*hb + m.  Both key
        // blocks advance together (four independent accumulators); fragments
        // are loaded two k-steps ahead of the MFMAs that use them.
        f32x4 sacc[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}},
                            {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
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
            sacc[0][0] = mfma_bf16(kf[c][0], qf[0][ks], sacc[0][0]);
            sacc[0][1] = mfma_bf16(kf[c][0], qf[1][ks], sacc[0][1]);
            sacc[1][0] = mfma_bf16(kf[c][1], qf[0][ks], sacc[1][0]);
            sacc[1][1] = mfma_bf16(kf[c][1], qf[1][ks], sacc[1][1]);
            if ((ks & 1) == 0) dma(nxt, nid, ks >> 1);  // loads 0..8 at the even steps
            __builtin_amdgcn_sched_barrier(0);
        }

        const int ids[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
        bool ok[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ok[i] = (unsigned)ids[i] < (unsigned)N;
        bf16x8 pa[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            // x = s * scale in base 2 (-inf for invalid slots); products are
            // never signalling NaNs, so the maxima need no canonicalisation
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = ok[i] ? sacc[i >> 2][hb][i & 3] * scale_log2 : -__builtin_inff();
            float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                             fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            // per-lane bookkeeping; the max over the head's four lane groups is
            // only needed to fix the reference on the first tile with a valid key
            if (m_ref[hb] == -__builtin_inff()) {
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                m_ref[hb] = mx;  // O and l are still 0
            }
            m_all[hb] = fmaxf(m_all[hb], mx);
            over |= mx > m_ref[hb] + REF_GAP;
            // exp2(-inf - m) = 0 for invalid slots; a head with no valid key so
            // far (m_ref = -inf) subtracts 0 instead, so its weights stay 0.
            // v_exp_f32 without range reduction: the argument is at most
            // REF_GAP (larger ones make the pass rerun) and results below the
            // normal range flush to 0, which the weights can afford.
            const float mr = m_ref[hb] == -__builtin_inff() ? 0.f : m_ref[hb];
            float p[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                p[i] = __builtin_amdgcn_exp2f(x[i] - mr);
                l_part[hb] += p[i];
            }
            pa[hb] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                            (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        }
        // P V, V fragments read two steps ahead
        auto vfrag = [&](int nv) __attribute__((always_inline)) -> bf16x8 {
            const int j = nv & 7, hi = 256 * (nv >> 3);
            const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + tr_off[j] + hi));
            const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(st + tr_off[j] + hi + 16 * LAT));
            const uint4 vv = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 0, 1)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 2, 3))};
            return as_bf16x8(vv);
        };
        bf16x8 vf[3];
        vf[0] = vfrag(0);
        vf[1] = vfrag(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nv = 0; nv < DV / 16; ++nv) {
            if (nv + 2 < DV / 16) vf[(nv + 2) % 3] = vfrag(nv + 2);
            o[0][nv] = mfma_bf16(pa[0], vf[nv % 3], o[0][nv]);
            o[1][nv] = mfma_bf16(pa[1], vf[nv % 3], o[1][nv]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // one ring step: wait for tile `it` (the loads of tiles it+1 and it+2 may
    // stay in flight), publish it with a barrier (which also tells every wave
    // that the stage read at it-1 is free), then multiply tile it while
    // refilling that stage with tile it+3
    auto step = [&](uint8_t* cur, uint8_t* nxt, int it) __attribute__((always_inline)) {
        if (it >= n_tiles) return;
        DSA_WAIT_VM(2 * DMA_PER_TILE);
        // a barrier that is also a compiler memory barrier (no LDS access moves
        // across it) but, unlike __syncthreads(), waits for no global loads
        // (its own earlier LDS reads are finished first, so no stage a
        // wave is still reading gets refilled)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        compute(cur, it, nxt);
    };

    // the first pass's ring prologue; then all of Q (k = 8*(l/16)+j within
    // each 32-wide step of d, loaded with the slot indices) is in registers
    // before the loop: the waits the compiler would otherwise place at Q's
    // first uses inside the loop would also wait for the gather loads it
    // does not know about
    issue(st0, 0);
    issue(st1, 1);
    issue(st2, 2);
    DSA_WAIT_VM(0);

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
            for (int i = 0; i < DV / 16; ++i) o[hb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            l_part[hb] = 0.f;
            m_ref[hb] = pass == 0 ? -__builtin_inff() : m_all[hb];
            if (pass == 0) m_all[hb] = -__builtin_inff();
        }
        if (pass == 1) {
            issue(st0, 0);
            issue(st1, 1);
            issue(st2, 2);
        }
        for (int it = 0; it < n_tiles; it += 4) {
            step(st0, st3, it);
            step(st1, st0, it + 1);
            step(st2, st1, it + 2);
            step(st3, st2, it + 3);
        }
        DSA_WAIT_VM(0);  // the loads past the last tile land before the stages are reused
        if (pass == 1) break;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {  // per-lane maxima -> max of the head
            m_all[hb] = fmaxf(m_all[hb], __shfl_xor(m_all[hb], 16, 64));
            m_all[hb] = fmaxf(m_all[hb], __shfl_xor(m_all[hb], 32, 64));
        }
        if (__any(over) && lane == 0) atomicOr(&s_redo, 1);
        __syncthreads();
        if (s_redo == 0) break;
    }

    // ---- finish: exp-sums per head, then per O row
    const int h0 = 32 * wave;
    float lo[2][4], l_tot[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        float lt = l_part[hb] + __shfl_xor(l_part[hb], 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        l_tot[hb] = lt;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[hb][i] = __shfl(lt, 4 * g + i, 64);
    }
    if (PARTIAL) {
        // this split's (max, exp-sum) per head; its O rows go out normalised
        const size_t pbase = (row * nsplit + split) * H;
        if (g == 0)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                part_ml[(pbase + h0 + 16 * hb + m) * 2 + 0] = m_ref[hb];
                part_ml[(pbase + h0 + 16 * hb + m) * 2 + 1] = l_tot[hb];
            }
    } else if (lse != nullptr && g == 0) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
            lse[row * H + h0 + 16 * hb + m] =
                l_tot[hb] > 0.f ? (m_ref[hb] + log2f(l_tot[hb])) * kLn2 : -__builtin_inff();
    }
    // normalise, stage the wave's 32 x 512 bf16 block (32 KiB) in its own ring
    // stage and store it with 16-byte writes
    __syncthreads();
    uint8_t* stage = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
    uint16_t* ob = reinterpret_cast<uint16_t*>(stage);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        float inv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) inv[i] = lo[hb][i] > 0.f ? 1.f / lo[hb][i] : 0.f;
#pragma unroll
        for (int nv = 0; nv < DV / 16; ++nv)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ob[(16 * hb + 4 * g + i) * DV + 16 * nv + m] =
                    __builtin_bit_cast(uint16_t, (__bf16)(o[hb][nv][i] * inv[i]));
    }
    __syncthreads();
    uint16_t* dst = PARTIAL ? part_o + ((row * nsplit + split) * H + h0) * DV : out + (row * H + h0) * DV;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        const int c = r * 64 + lane;  // 16-byte chunk of the wave's block
        *reinterpret_cast<uint4*>(dst + c * 8) = *reinterpret_cast<const uint4*>(ob + c * 8);
    }
}

// Merge the per-split partials (normalised bf16 O rows, max, exp-sum): the
// split weights are sum_s * 2^(max_s - M).  One thread per 4 output columns
// of one head, 4 heads per workgroup.
__global__ __launch_bounds__(512) void attn_combine(const uint16_t* __restrict__ part_o,
                                                   const float* __restrict__ part_ml,
                                                   uint16_t* __restrict__ out, float* __restrict__ lse,
                                                   int nsplit, int rows) {
    // 32 workgroups (4 heads each) per row.  When the row count is a multiple
    // of 8, the attention kernel ran rows [x*rows/8, (x+1)*rows/8) on XCD x;
    // merge them there too, where their partials were just written.
    unsigned r, hg;
    if ((rows & 7) == 0) {
        const unsigned x = blockIdx.x & 7u, j = blockIdx.x >> 3;
        r = x * (unsigned)(rows >> 3) + (j >> 5);
        hg = j & 31u;
    } else {
        r = blockIdx.x >> 5;
        hg = blockIdx.x & 31u;
    }
    const size_t row = r;
    const int h = hg * 4 + (threadIdx.x >> 7);
    const int v = (threadIdx.x & 127) * 4;
    // every load first (at most 8 slot ranges: k <= 2048, >= 256 slots each),
    // then the arithmetic
    constexpr int MAXS = 8;
    float mv[MAXS], lv[MAXS];
    uint2 xv[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
        if (s < nsplit) {
            const size_t pb = (row * nsplit + s) * H + h;
            mv[s] = part_ml[pb * 2];
            lv[s] = part_ml[pb * 2 + 1];
            xv[s] = *reinterpret_cast<const uint2*>(part_o + pb * DV + v);
        } else {
            mv[s] = -__builtin_inff();
            lv[s] = 0.f;
            xv[s] = uint2{0u, 0u};
        }
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < MAXS; ++s) M = fmaxf(M, mv[s]);
    float L = 0.f;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
        const float f = mv[s] == -__builtin_inff() ? 0.f : lv[s] * exp2f(mv[s] - M);
        L += f;
        acc.x += __uint_as_float(xv[s].x << 16) * f;
        acc.y += __uint_as_float(xv[s].x & 0xffff0000u) * f;
        acc.z += __uint_as_float(xv[s].y << 16) * f;
        acc.w += __uint_as_float(xv[s].y & 0xffff0000u) * f;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint2 pk;
    pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.x * inv)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.y * inv)) << 16);
    pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.z * inv)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(out + (row * H + h) * DV + v) = pk;
    if (lse != nullptr && v == 0) lse[row * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -__builtin_inff();
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
    return align_up((size_t)rows * s * H_ * d_v * sizeof(uint16_t)) +
           align_up((size_t)rows * s * H_ * 2 * sizeof(float));
}

dsa_status launch_attn_bf16(const void* q, const void* kv, const int32_t* idx, void* out,
                            float* lse, int B, int T, int N, int k, float sm_scale,
                            void* workspace, hipStream_t stream) {
    if (k > SLOTS) return DSA_ERR_UNSUPPORTED;
    if (T > 65535 || B > 65535) return DSA_ERR_UNSUPPORTED;
    if ((size_t)N * (2 * DQK) >= 0x80000000ull) return DSA_ERR_UNSUPPORTED;  // 32-bit gather offsets
    const long long rows = (long long)B * T;
    const int s = attn_num_splits((int)std::min<long long>(rows, 1 << 30), k);
    const float scale_log2 = sm_scale * kLog2e;
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(kv);
    auto* oo = static_cast<uint16_t*>(out);
    if (s <= 1) {
        sparse_mla_attn_bf16<false><<<dim3((unsigned)rows), NTA, 0, stream>>>(
            qq, kk, idx, oo, lse, nullptr, nullptr, T, N, k, 1, k, scale_log2);
        return launch_status();
    }
    const int per = ((k + s - 1) / s + TK - 1) / TK * TK;
    const int s_eff = (k + per - 1) / per;
    uint16_t* part_o = static_cast<uint16_t*>(workspace);
    float* part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              align_up((size_t)rows * s * H * DV * sizeof(uint16_t)));
    sparse_mla_attn_bf16<true><<<dim3((unsigned)(rows * s_eff)), NTA, 0, stream>>>(
        qq, kk, idx, oo, lse, part_o, part_ml, T, N, k, s_eff, per, scale_log2);
    dsa_status st = launch_status();
    if (st != DSA_OK) return st;
    attn_combine<<<dim3((unsigned)rows * (H / 4)), 512, 0, stream>>>(part_o, part_ml, oo, lse, s_eff,
                                                                    (int)rows);
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
