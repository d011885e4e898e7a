// Sparse MLA attention in MQA mode on gfx950.
//
// Method ("Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture: DSA
// (§2.1)"): u_t = Attn(h_t, {c_s : I[t,s] in Top-k(I[t,:])}); under "DSA
// under MLA (MQA Mode)" one latent vector c_s (576 wide: 512 latent + 64
// rope) per selected token is shared by all 128 query heads, and the value
// is its 512-wide latent part.
//
// bf16 path: one workgroup (4 waves, one per SIMD) per query token and slot
// range.  The selected latent rows are gathered 32 at a time (a tile)
// straight into LDS with direct-to-LDS loads (no registers in flight)
// through a ring of four 36 KiB stages; the loads of tile i+2 are issued
// between the key-product MFMAs of tile i.  Latent rows are stored with
// their 16-byte chunks swizzled so that both the key-product fragment reads
// and the transposed value reads are free of bank conflicts.
//
// Per tile:
//   S^T[key, head] = K[key, :] . Q[head, :]    wave w: heads 32w..32w+31,
//     36 bf16 MFMA 32x32x16 in two accumulator chains (A = key rows from
//     LDS, B = the wave's Q in VGPRs); S^T puts one head per lane column,
//     the layout the P operand of the value product needs
//   softmax in base 2 against a fixed reference max per head (the max of
//     the first tile with a valid key): exp2(x - m_ref) may grow to
//     2^REF_GAP, which fp32 sums and bf16 weights carry without loss of
//     relative precision, so the accumulator is never rescaled; a tile that
//     exceeds the reference by more than REF_GAP makes the workgroup redo
//     the pass against the exact max it recorded
//   P: each wave's 32 heads of weights (bf16) into a shared 8 KiB LDS buffer
//   O[head, v] += P[head, key] V[key, v]      wave w: value columns
//     128w..128w+127 of all 128 heads, 4 x 4 blocks x 2 k steps = 32 bf16
//     MFMA 32x32x16 (V^T fragments from the latent rows in LDS through
//     ds_read_b64_tr_b16 transposed reads; their key order matches the P
//     operand's)
// The O accumulator (128 heads x 128 fp32 columns per wave) lives in AGPRs.
// Batches with fewer rows than CUs split the slots over several
// workgroups; each writes its O rows normalised in bf16 with its per-head
// (max, exp-sum), and attn_combine merges them.
#include <type_traits>

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

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The key product's accumulator chain in VGPRs.  With the whole AGPR file
// holding the 32 x 512 fp32 output accumulator, the compiler would otherwise
// give this chain AGPRs too (every MFMA gets the AGPR form when a kernel
// uses AGPRs) and shuttle output blocks between the two register files.
// first: D = A B (no accumulator read); next: D += A B (the back-to-back
// dependent accumulation the MFMA pipe forwards); last: D += A B followed by
// 24 wait states before any other instruction may read D (an XDL result read
// by VALU or memory instructions needs up to passes + 3 = 19 of them).
__device__ __forceinline__ void qk_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_next(f32x16& d, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(d)
                 : "v"(a), "v"(b));
}

// LDS layout of a gathered tile: latent row r (1 KiB) keeps its 16-byte
// chunk c in slot c ^ lat_swz(r); the rope parts (128 B per row) follow the
// 32 latent rows, chunk c of row r in slot c ^ rope_swz(r).
//  * key-fragment reads (ds_read_b128, 16 lanes per pass): 16 consecutive
//    rows at one chunk -- lat_swz is a permutation of 0..15 on any 16
//    consecutive rows, and rope_swz on rows of one parity;
//  * transposed value reads (ds_read_b64_tr_b16, 32 lanes per pass): 4
//    consecutive rows x 4 consecutive chunks -- lat_swz gives the 4 rows
//    different multiples of 4.
// Both land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int lat_swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

// P of one tile as the value product's A operands: 4 head blocks x 2 k steps
// x 64 lanes x 16 bytes.
constexpr int PBYTES = NWV * 2 * 64 * 16;

template <bool PARTIAL, bool NEG>
__global__ __launch_bounds__(NTA) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml, int T, int N, int k, int nsplit, int slots_per_split,
    float scale_log2) {
    // four ring stages; tile t lives in stage t % 4
    __shared__ __attribute__((aligned(16))) uint8_t ring[4 * STAGE];
    __shared__ __attribute__((aligned(16))) int32_t sidx[SLOTS];
    // the current tile's P, shared by the four waves; outside the tile loop
    // the same bytes hold the workgroup's scalars (setup, pass end) and the
    // exp-sums of all heads (finish)
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[PBYTES];
    int* const s_last = reinterpret_cast<int*>(pbuf);
    int* const s_redo = reinterpret_cast<int*>(pbuf) + 1;
    unsigned* const s_notfull = reinterpret_cast<unsigned*>(pbuf) + 4;  // tiles with an invalid slot
    float* const s_l = reinterpret_cast<float*>(pbuf);

    // (split batches only: causal prefill rows differ in length, and giving
    // each XCD a contiguous range of them would unbalance the XCDs)
    const unsigned item = PARTIAL ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const int split = (int)(item % (unsigned)nsplit);
    const size_t row = item / (unsigned)nsplit;
    const int b = (int)(row / (unsigned)T);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // 32x32 MFMA lane roles: column hl (a head, a key row or a value column),
    // half hh (which 8 of the 16 k indices the lane holds)
    const int hl = lane & 31, hh = lane >> 5;
    const int slot0 = split * slots_per_split;
    const int nslots = max(0, min(k - slot0, slots_per_split));
    const uint16_t* __restrict__ kv_b = kv + (size_t)b * N * DQK;

    // ---- slot indices of this workgroup; the last valid one
    if (tid == 0) *s_last = -1;
    if (tid < SLOTS / TK / 32) s_notfull[tid] = 0;
    __syncthreads();
    int my_last = -1;
    const int nslots_pad = (nslots + TK - 1) / TK * TK;
    // this wave's 32 query heads as B operands: lane (hl, hh) holds head
    // 32*wave + hl, features 16*ks + 8*hh .. +7
    bf16x8 qf[DQK / 16];
    {
        // all of a thread's index loads are issued before the first is
        // waited for (a loop that stores each index as it arrives waits for
        // one memory round trip per iteration), and Q's loads right behind
        // them, so that Q arrives while the indices are used
        constexpr int PER = (SLOTS + NTA - 1) / NTA;
        int id[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTA;
            id[j] = i < nslots ? idx[row * k + slot0 + i] : -1;
        }
        const uint16_t* qh = q + (row * H + 32 * wave + hl) * DQK + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks)
            qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qh + 16 * ks));
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTA;
            if (i < nslots_pad) {
                sidx[i] = id[j];
                if (id[j] >= 0 && id[j] < N) my_last = i;
                else atomicOr(&s_notfull[i / (32 * TK)], 1u << ((i / TK) & 31));
            }
        }
    }
    if (my_last >= 0) atomicMax(s_last, my_last);

    __syncthreads();
    const int last = *s_last;
    const unsigned nf0 = s_notfull[0], nf1 = s_notfull[1];  // (read before the first P is written)
    const int n_tiles = (last + TK) / TK;  // 0 when no slot is valid
    // rows of invalid slots are loaded from a selected row (their weight is 0)
    const int dummy = last >= 0 ? sidx[last] : 0;

    // Softmax without rescaling the accumulator: the reference max m_ref of
    // the lane's head is the max of the first tile with a valid key, and
    // later exponentials exp2(x - m_ref) may grow up to 2^REF_GAP, which fp32
    // accumulators and bf16 weights hold without loss of relative precision.
    // A tile that exceeds the reference by more than REF_GAP flags the
    // workgroup, which then reruns the pass with m_ref = the exact max it
    // recorded (so every exponential is <= 1).
    //
    // O: the wave's 128 value columns 128*wave .. +127 of all 128 heads,
    // 4 x 4 blocks of 32 heads x 32 columns (block (hb, cb) in o[hb][cb]).
    f32x16 o[4][4];
    float m_ref = -__builtin_inff(), m_all = -__builtin_inff(), l_part = 0.f;
    bool over = false;

    // Per-lane LDS offsets inside a stage (the same for every tile).
    // Key fragment of step ks (A operand: key row hl, features 16ks + 8hh):
    // latent chunk 2ks + hh (ks < 32) in slot (2ks + hh) ^ lat_swz(hl)
    // = 256*(ks/8) + 32*((ks%8) ^ (f>>1)) + 16*((hh ^ f) & 1); rope chunk
    // 2(ks-32) + hh (ks >= 32) in slot (2(ks-32) + hh) ^ rope_swz(hl).
    int k_off[8], r_off[4];
    {
        const int f = lat_swz(hl), fr = rope_swz(hl);
#pragma unroll
        for (int j = 0; j < 8; ++j) k_off[j] = hl * LAT + 16 * ((2 * j + hh) ^ f);
#pragma unroll
        for (int j = 0; j < 4; ++j) r_off[j] = TK * LAT + hl * ROPE + 16 * ((2 * j + hh) ^ fr);
    }
    // Value fragment of k step kk and column block nb (B operand: column
    // 32nb + hl, the eight keys of half hh in the order the S^T accumulator
    // holds them: 16kk + 4hh + {0..3}, then 16kk + 8 + 4hh + {0..3}).  Two
    // transposed reads: in each 16-lane group g (= 2hh + gc), lane m reads 8
    // bytes of row 16kk + 8j + 4hh + m/4 at columns 32nb + 16gc + 4(m%4),
    // i.e. chunk 4nb + 2gc + (m%4)/2, and receives column 32nb + 16gc + m of
    // the four rows.  lat_swz of those rows is 4(m/4) + ((2j + hh) & 3),
    // independent of kk; slot = 16*(nb/4) + ((4(nb%4) + 2gc + (m%4)/2) ^ f).
    // The wave's column blocks are nb = 4*wave + cb: the 256-byte group
    // nb/4 = wave, and nb%4 = cb.
    int v_off[2][4];
    {
        const int m = lane & 15, gc = (lane >> 4) & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 8 * j + 4 * hh + (m >> 2);
            const int f = lat_swz(r);
#pragma unroll
            for (int nq = 0; nq < 4; ++nq)
                v_off[j][nq] = r * LAT + 256 * wave + 16 * ((4 * nq + 2 * gc + ((m & 3) >> 1)) ^ f) + 8 * (m & 1);
        }
    }
    const unsigned ring_base = lds_addr(ring);
    auto stage_of = [&](int tile) __attribute__((always_inline)) -> const uint8_t* {
        return ring + (tile & 3) * STAGE;
    };

    // direct-to-LDS gather of one tile: wave w brings latent rows 8w..8w+7
    // (one 1 KiB row per instruction, lane l fetching chunk l ^ lat_swz(r))
    // and the rope parts of rows 8w..8w+7 (lane l: row 8w+l/8, chunk
    // (l%8) ^ rope_swz(row)); 9 loads per wave and tile.  The loads go
    // through a buffer resource over this sequence's rows (the base stays in
    // SGPRs; the row offset of a latent load is a scalar).  A tile at or past
    // n_tiles is still "loaded", with offsets beyond the resource's range:
    // such loads touch no memory, so every tile issues the same number of
    // loads and the ring's wait counts do not depend on the position.
    // gather_id() looks the rows up (lane l: row 8w + l/8); dma(u) issues
    // load u.
    const i32x4 kv_rsrc = buffer_rsrc(kv_b, (unsigned)N * (unsigned)(2 * DQK));
    const int lane16 = lane << 4;
    auto gather_id = [&](int tile) __attribute__((always_inline)) {
        if (tile >= n_tiles) return -1;
        const int r = 8 * wave + (lane >> 3);
        int id = sidx[tile * TK + r];
        if (id < 0 || id >= N) id = dummy;
        return id;
    };
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto dma = [&](int tile, int id, int u) __attribute__((always_inline)) {
        const unsigned st = ring_base + (unsigned)((tile & 3) * STAGE);
        if (u < 8) {
            const int ru = 8 * wave_s + u;
            const int idu = __builtin_amdgcn_readlane(id, 8 * u);
            const unsigned vo = idu < 0 ? 0x80000000u : (unsigned)(lane16 ^ (lat_swz(ru) << 4));
            load_lds16(kv_rsrc, st + ru * LAT, vo, (unsigned)max(idu, 0) * (2 * DQK));
        } else {
            const int r = 8 * wave + (lane >> 3);
            const unsigned vo = id < 0 ? 0x80000000u
                                       : (unsigned)id * (2 * DQK) + 1024 + 16 * ((lane & 7) ^ rope_swz(r));
            load_lds16(kv_rsrc, st + TK * LAT + wave_s * 1024, vo, 0u);
        }
    };
    auto issue = [&](int tile) __attribute__((always_inline)) {
        const int id = gather_id(tile);
#pragma unroll
        for (int u = 0; u < DMA_PER_TILE; ++u) dma(tile, id, u);
    };
    auto kfrag = [&](const uint8_t* st, int ks) __attribute__((always_inline)) -> bf16x8 {
        const uint8_t* p = ks < 32 ? st + k_off[ks & 7] + 256 * (ks >> 3) : st + r_off[ks - 32];
        return as_bf16x8(*reinterpret_cast<const uint4*>(p));
    };
    // a workgroup barrier that is also a compiler memory barrier (no LDS
    // access moves across it) but, unlike __syncthreads(), waits for no
    // global loads (its own earlier LDS reads are finished first, so no stage
    // or P a wave is still reading gets overwritten)
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // S^T of tile `tile` into sacc; the loads of tile `tile + 2` are spread
    // over its steps.  Register i of the accumulator holds key
    // 8(i/4) + 4hh + i%4 of head hl.
    auto qk = [&](int tile, f32x16& sacc) __attribute__((always_inline)) {
        const uint8_t* st = stage_of(tile);
        const int nid = gather_id(tile + 2);
        // two accumulator chains (even and odd steps): a dependent MFMA waits
        // for its predecessor's result, so one chain would run the MFMA
        // pipe at about two thirds of its rate
        f32x16 s_odd;
        constexpr int KD = 2;  // prefetch distance
        bf16x8 kf[KD + 1];
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) kf[ks] = kfrag(st, ks);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks) {
            if (ks + KD < DQK / 16) kf[(ks + KD) % (KD + 1)] = kfrag(st, ks + KD);
            f32x16& acc = (ks & 1) ? s_odd : sacc;
            const bf16x8& kcur = kf[ks % (KD + 1)];
            if (ks < 2) qk_first(acc, kcur, qf[ks]);
            else if (ks + 1 < DQK / 16) qk_next(acc, kcur, qf[ks]);
            else qk_last(acc, kcur, qf[ks]);
            if ((ks & 3) == 0) dma(tile + 2, nid, ks >> 2);  // loads 0..8 at steps 0, 4, .., 32
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] += s_odd[i];
    };

    // Softmax of tile `tile` (S^T in s, turned into the weights in place), in
    // pieces so that it can run in the shadow of other work.  The max runs
    // over all 32 raw logits: a slot that is not valid gathered the dummy
    // row, the last valid row of this workgroup, so its logit repeats one of
    // the valid ones and the max is that of the valid slots, exactly.  With
    // a non-negative scale max(s * scale) = max(s) * scale (s * scale is
    // monotonic in s; NEG: -max(-s) * scale for a negative one); each weight
    // is exp2(fma(s, scale, -m)), and the weights of slots that are not valid
    // are set to 0.  Only tiles with an invalid slot read the slot indices.
    // The weights end up as bf16 A operands in pa (k step kk = accumulator
    // registers 8kk .. 8kk+7).
    struct Soft {
        unsigned okm;
        float mx, mr;
    };
    auto soft_begin = [&](int tile, Soft& sf) __attribute__((always_inline)) {
        sf.mx = -__builtin_inff();
        sf.mr = 0.f;
        unsigned okm = 0xffffu;
        if ((((tile < 32) ? nf0 : nf1) >> (tile & 31)) & 1u) {
            // validity of this lane's keys 8j + 4hh + {0..3}, j = 0..3, as a mask
            okm = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int4 iv = *reinterpret_cast<const int4*>(&sidx[tile * TK + 8 * j + 4 * hh]);
                okm |= ((unsigned)iv.x < (unsigned)N ? 1u : 0u) << (4 * j);
                okm |= ((unsigned)iv.y < (unsigned)N ? 1u : 0u) << (4 * j + 1);
                okm |= ((unsigned)iv.z < (unsigned)N ? 1u : 0u) << (4 * j + 2);
                okm |= ((unsigned)iv.w < (unsigned)N ? 1u : 0u) << (4 * j + 3);
            }
        }
        sf.okm = okm;
    };
    auto soft_piece = [&](int j, f32x16& sv, Soft& sf, bf16x8* pa) __attribute__((always_inline)) {
        if (j < 8) {
            // products are never signalling NaNs, so the maxima need no
            // canonicalisation
            sf.mx = NEG ? fmaxf(sf.mx, fmaxf(-sv[2 * j], -sv[2 * j + 1]))
                        : fmaxf(sf.mx, fmaxf(sv[2 * j], sv[2 * j + 1]));
        } else if (j == 8) {
            // per-lane bookkeeping; the head's max over both lane halves is
            // only needed to fix the reference on the first tile
            float mx = NEG ? sf.mx * -scale_log2 : sf.mx * scale_log2;
            if (m_ref == -__builtin_inff()) {
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                m_ref = mx;  // O and l are still 0
            }
            m_all = fmaxf(m_all, mx);
            over |= mx > m_ref + REF_GAP;
            // v_exp_f32 without range reduction: the argument is at most
            // REF_GAP (larger ones make the pass rerun) and results below the
            // normal range flush to 0, which the weights can afford.
            sf.mr = m_ref;
        } else if (j < 17) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * (j - 9) + e;
                const float pw = __builtin_amdgcn_exp2f(fmaf(sv[i], scale_log2, -sf.mr));
                sv[i] = (sf.okm >> i) & 1u ? pw : 0.f;
                l_part += sv[i];
            }
        } else if (j < 19) {
            const int kk = j - 17;
            pa[kk] = bf16x8{(__bf16)sv[8 * kk + 0], (__bf16)sv[8 * kk + 1], (__bf16)sv[8 * kk + 2],
                            (__bf16)sv[8 * kk + 3], (__bf16)sv[8 * kk + 4], (__bf16)sv[8 * kk + 5],
                            (__bf16)sv[8 * kk + 6], (__bf16)sv[8 * kk + 7]};
        }
    };

    // The wave's P (its 32 heads = head block `wave`) into the shared buffer:
    // A operand (head block hb, k step kk) of lane l at 16-byte slot
    // (2 hb + kk) * 64 + l, exactly the registers the softmax left in lane l.
    auto write_p = [&](const bf16x8* pa) __attribute__((always_inline)) {
        uint4* pw = reinterpret_cast<uint4*>(pbuf) + 2 * wave * 64 + lane;
        pw[0] = __builtin_bit_cast(uint4, pa[0]);
        pw[64] = __builtin_bit_cast(uint4, pa[1]);
    };

    // O[head, v] += P V over tile `tile` for the wave's 128 value columns and
    // all four head blocks (P from the shared buffer); when SOFT, the pieces
    // of the next tile's softmax (on sn, into pn) run between the MFMAs.
    // Value fragments of k step 0 are read first, those of k step 1 during
    // the second half of step 0; each P fragment one head block ahead.
    auto pv = [&](int tile, auto soft_t, f32x16& sn, Soft& sf, bf16x8* pn) __attribute__((always_inline)) {
        constexpr bool SOFT = decltype(soft_t)::value;
        const uint8_t* st = stage_of(tile);
        const uint4* pr = reinterpret_cast<const uint4*>(pbuf) + lane;
        auto vfrag = [&](int kk, int cb) __attribute__((always_inline)) -> bf16x8 {
            const uint8_t* base = st + kk * 16 * LAT;
            const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + v_off[0][cb]));
            const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + v_off[1][cb]));
            const uint4 vv = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 0, 1)),
                              __builtin_bit_cast(uint32_t, __builtin_shufflevector(c, c, 2, 3))};
            return as_bf16x8(vv);
        };
        auto afrag = [&](int hb, int kk) __attribute__((always_inline)) -> bf16x8 {
            return as_bf16x8(pr[(2 * hb + kk) * 64]);
        };
        bf16x8 vb[2][4], pf[2];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) vb[0][cb] = vfrag(0, cb);
        pf[0] = afrag(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                const int step = 4 * kk + hb;
                if (step + 1 < 8) pf[(step + 1) & 1] = afrag((hb + 1) & 3, kk + ((hb + 1) >> 2));
                if (kk == 0 && hb == 2) {
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) vb[1][cb] = vfrag(1, cb);
                }
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    o[hb][cb] = mfma32(pf[step & 1], vb[kk][cb], o[hb][cb]);
                    const int s = 4 * step + cb;
                    if (SOFT && s < 19) soft_piece(s, sn, sf, pn);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // the first pass's ring prologue; then all of Q (loaded with the slot
    // indices) is in registers before the loop: the waits the compiler would
    // otherwise place at Q's first uses inside the loop would also wait for
    // the gather loads it does not know about
    issue(0);
    issue(1);
    DSA_WAIT_VM(0);

    // Pipeline of a pass: tile t's S^T on the MFMA pipe; then tile t-1's
    // P V on the MFMA pipe with tile t's softmax on the VALU in its shadow;
    // then, once every wave has read tile t-1's P, tile t's P goes into the
    // shared buffer.  Tile t + 2 is gathered during tile t's S^T into the
    // stage of tile t-2, which every wave has finished with at tile t's
    // barrier.
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[hb][cb][e] = 0.f;
        l_part = 0.f;
        m_ref = pass == 0 ? -__builtin_inff() : m_all;
        if (pass == 0) m_all = -__builtin_inff();
        if (pass == 1) {
            issue(0);
            issue(1);
        }
        if (n_tiles > 0) {
            f32x16 s;
            Soft sf;
            bf16x8 pa[2];
            // tile 0 (tile 1's loads may stay in flight)
            DSA_WAIT_VM(DMA_PER_TILE);
            lds_barrier();
            qk(0, s);
            soft_begin(0, sf);
#pragma unroll
            for (int j = 0; j < 19; ++j) soft_piece(j, s, sf, pa);
            write_p(pa);
            for (int it = 1; it < n_tiles; ++it) {
                DSA_WAIT_VM(DMA_PER_TILE);
                lds_barrier();  // tile it is in, and every wave's P of tile it-1
                qk(it, s);
                soft_begin(it, sf);
                pv(it - 1, std::true_type{}, s, sf, pa);
                lds_barrier();  // every wave is done with tile it-1's P
                write_p(pa);
            }
            lds_barrier();
            pv(n_tiles - 1, std::false_type{}, s, sf, pa);
        }
        DSA_WAIT_VM(0);  // the loads past the last tile land before the stages are reused
        if (pass == 1) break;
        m_all = fmaxf(m_all, __shfl_xor(m_all, 32, 64));  // per-lane maxima -> max of the head
        // (s_redo shares the P buffer: every wave is done with it first)
        __syncthreads();
        if (tid == 0) *s_redo = 0;
        __syncthreads();
        if (__any(over) && lane == 0) atomicOr(s_redo, 1);
        __syncthreads();
        const bool redo = *s_redo != 0;
        __syncthreads();
        if (!redo) break;
    }

    // ---- finish: exp-sum of the lane's head (both halves); every head's
    // exp-sum through LDS to the waves that hold its O columns
    const int h0 = 32 * wave;
    const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
    if (PARTIAL) {
        // this split's (max, exp-sum) per head; its O rows go out normalised
        const size_t pbase = (row * nsplit + split) * H;
        if (hh == 0) {
            part_ml[(pbase + h0 + hl) * 2 + 0] = m_ref;
            part_ml[(pbase + h0 + hl) * 2 + 1] = l_tot;
        }
    } else if (lse != nullptr && hh == 0) {
        lse[row * H + h0 + hl] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -__builtin_inff();
    }
    __syncthreads();  // (s_l shares the P buffer)
    if (hh == 0) s_l[h0 + hl] = l_tot;
    __syncthreads();
    // o[hb][cb] register i holds head 32hb + 8(i/4) + 4hh + i%4, column
    // 128 wave + 32 cb + hl.  Normalised, rounded to bf16 and stored straight
    // from registers in column pairs: adjacent lanes (hl even / odd) trade
    // one value by DPP so that the even lane holds columns hl, hl+1 of head
    // i and the odd lane columns hl-1, hl of head i+1; each store then writes
    // four 64-byte row segments.
    uint16_t* dst = PARTIAL ? part_o + (row * nsplit + split) * H * DV : out + row * H * DV;
    const bool odd = (hl & 1) != 0;
    // a buffer resource over the row's H x DV outputs: the lane's part of the
    // byte offset in a VGPR, the head block / register / column block part a
    // scalar constant per store
    const auto o_rs = __builtin_amdgcn_make_buffer_rsrc(dst, 0, H * DV * 2, 0x00020000);
    const int o_voff = ((4 * hh + (odd ? 1 : 0)) * DV + 128 * wave + (hl & ~1)) * 2;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const float4 lv = *reinterpret_cast<const float4*>(&s_l[32 * hb + 8 * i4 + 4 * hh]);
            const float la[4] = {lv.x, lv.y, lv.z, lv.w};
            float inv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) inv[e] = la[e] > 0.f ? 1.f / la[e] : 0.f;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const float x0 = o[hb][cb][4 * i4 + e] * inv[e];
                    const float x1 = o[hb][cb][4 * i4 + e + 1] * inv[e + 1];
                    const float send = odd ? x0 : x1;
                    const float recv = __builtin_bit_cast(
                        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xf, 0xf, false));
                    const float lo = odd ? recv : x0, hi = odd ? x1 : recv;
                    const uint32_t pk = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
                    __builtin_amdgcn_raw_buffer_store_b32(pk, o_rs, o_voff,
                                                          ((32 * hb + 8 * i4 + e) * DV + 32 * cb) * 2, 0);
                }
            }
        }
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
    // (a negative softmax scale takes the kernel copy that tracks max(-s))
    const bool neg = scale_log2 < 0.f;
    if (s <= 1) {
        if (neg)
            DSA_TIMED("sparse_mla_attn_bf16<false, true>", stream,
                      sparse_mla_attn_bf16<false, true><<<dim3((unsigned)rows), NTA, 0, stream>>>(
                          qq, kk, idx, oo, lse, nullptr, nullptr, T, N, k, 1, k, scale_log2));
        else
            DSA_TIMED("sparse_mla_attn_bf16<false, false>", stream,
                      sparse_mla_attn_bf16<false, false><<<dim3((unsigned)rows), NTA, 0, stream>>>(
                          qq, kk, idx, oo, lse, nullptr, nullptr, T, N, k, 1, k, scale_log2));
        return launch_status();
    }
    const int per = ((k + s - 1) / s + TK - 1) / TK * TK;
    const int s_eff = (k + per - 1) / per;
    uint16_t* part_o = static_cast<uint16_t*>(workspace);
    float* part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              align_up((size_t)rows * s * H * DV * sizeof(uint16_t)));
    if (neg)
        DSA_TIMED("sparse_mla_attn_bf16<true, true>", stream,
                  sparse_mla_attn_bf16<true, true><<<dim3((unsigned)(rows * s_eff)), NTA, 0, stream>>>(
                      qq, kk, idx, oo, lse, part_o, part_ml, T, N, k, s_eff, per, scale_log2));
    else
        DSA_TIMED("sparse_mla_attn_bf16<true, false>", stream,
                  sparse_mla_attn_bf16<true, false><<<dim3((unsigned)(rows * s_eff)), NTA, 0, stream>>>(
                      qq, kk, idx, oo, lse, part_o, part_ml, T, N, k, s_eff, per, scale_log2));
    dsa_status st = launch_status();
    if (st != DSA_OK) return st;
    DSA_TIMED("attn_combine", stream,
              attn_combine<<<dim3((unsigned)rows * (H / 4)), 512, 0, stream>>>(part_o, part_ml, oo,
                                                                              lse, s_eff, (int)rows));
    return launch_status();
}

dsa_status launch_attn_f32(const float* q, const float* kv, const int32_t* idx, float* out,
                           float* lse, int B, int T, int N, int Hn, int d_qk, int d_v, int k,
                           float sm_scale, hipStream_t stream) {
    if (k > SLOTS || d_qk > 256 || Hn > 32) return DSA_ERR_UNSUPPORTED;
    if (B > 65535) return DSA_ERR_UNSUPPORTED;
    DSA_TIMED("sparse_attn_f32", stream,
              sparse_attn_f32<<<dim3(T, B), NTF, 0, stream>>>(q, kv, idx, out, lse, T, N, Hn, d_qk,
                                                              d_v, k, sm_scale));
    return launch_status();
}

}  // namespace dsa
