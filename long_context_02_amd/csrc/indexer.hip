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
#include <type_traits>

#include "indexer_math.h"
#include "topk_select.h"

namespace dsa {
namespace {

constexpr int NT = 256;    // threads per workgroup (4 waves)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBuf = 0x00020000;  // buffer resource word 3: raw (untyped) 32-bit data

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
__global__ __launch_bounds__(NTT) __attribute__((amdgpu_waves_per_eu(4))) void indexer_fp8_tiled(
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
        // cooperative staging: 512 16-byte chunks per tile, one per thread,
        // through buffer resources (the tile's key offset is a scalar; keys
        // at or past N read as zeros)
        const int c_key = tid >> 3, c_piece = tid & 7;
        // (byte counts and offsets are 32-bit: N < 2^24, checked on the host)
        const auto k_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(k_b), 0,
                                                            (int)((unsigned)N * DI), kRawBuf);
        const auto ks_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ks_b), 0, 4 * N, kRawBuf);
        const int k_voff = DI * c_key + 16 * c_piece;
        u32x4 r0;
        float rks = 0.f;
        auto fetch = [&](int s0) {
            r0 = __builtin_amdgcn_raw_buffer_load_b128(k_rs, k_voff, s0 * DI, 0);
            if (tid < TILE) rks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ks_rs, 4 * tid, 4 * s0, 0));
        };
        auto stage = [&](int buf) {
            *reinterpret_cast<u32x4*>(&lds_k[buf][c_key * ROWB + 16 * c_piece]) = r0;
            if (tid < TILE) lds_ks[buf][tid] = rks;
        };
        // score stores through a buffer over the workgroup's rows [t0, t_end):
        // per lane a fixed byte offset per row step, the tile's key offset a
        // scalar; stores to rows at or past t_end fall outside and are dropped
        const auto o_rs = __builtin_amdgcn_make_buffer_rsrc(out_b + (size_t)t0 * N, 0,
                                                            (int)(4u * (unsigned)(t_end - t0) * (unsigned)N), kRawBuf);
        int o_voff[QPW / 4];
#pragma unroll
        for (int j = 0; j < QPW / 4; ++j)
            o_voff[j] = (int)(4u * ((unsigned)(tw0 - t0 + 4 * j + (lane >> 4)) * (unsigned)N + 4u * (lane & 15)));

        // One tile: the scores of its 64 keys for the wave's queries into LDS,
        // then out as whole 256-byte row segments.  MASKED applies the causal
        // mask and the range checks; the leading tiles, whose keys every query
        // of the workgroup sees, skip them.
        auto tile = [&](int it, auto masked) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked)::value;
            const int s0 = s_begin + it * TILE;
            const int buf = it & 1;
            const bool more = it + 1 < n_tiles;
            if (more) fetch(s0 + TILE);
            float* ost = lds_o[wave];
            if (tw0 < t_end) {
                // Software pipelined over the tile's four 16-key steps and the
                // wave's two query groups: the MFMAs of (step j + 1, group g)
                // are issued right after the epilogue of (j, g) has read the
                // group's accumulators, so an epilogue never waits for a
                // product just issued and each group needs one accumulator set.
                constexpr int NSUB = TILE / 16;
                static_assert(GPW == 2, "two query groups per wave");
                i32x8 bfr[2];
                float kscr[2];
                f32x4 acc[GPW][2];
                auto ldb = [&](int sub) __attribute__((always_inline)) {
                    const uint8_t* src = &lds_k[buf][(16 * sub + m) * ROWB + 32 * kb];
                    bfr[sub & 1] = pack8(*reinterpret_cast<const uint4*>(src),
                                         *reinterpret_cast<const uint4*>(src + 16));
                    kscr[sub & 1] = lds_ks[buf][16 * sub + m];
                };
                auto mm = [&](int sub, int g) __attribute__((always_inline)) {
                    acc[g][0] = mfma_fp8(a[g][0], bfr[sub & 1]);
                    acc[g][1] = mfma_fp8(a[g][1], bfr[sub & 1]);
                };
                auto epi = [&](int sub, int g) __attribute__((always_inline)) {
                    const int key = 16 * sub + m;
                    float sc = head_sum(acc[g][0], acc[g][1], ws[g]) * kscr[sub & 1];
                    if (MASKED && s0 + key > q_offset + tw0 + 4 * g + kb) sc = -__builtin_inff();
                    ost[(4 * g + kb) * OST + key] = sc;
                };
                ldb(0);
                mm(0, 0);
                mm(0, 1);
                ldb(1);
#pragma unroll
                for (int sub = 0; sub < NSUB; ++sub) {
                    // (scheduling barriers keep this order: the compiler would
                    // otherwise move each epilogue next to the MFMAs it reads
                    // and wait for them)
                    __builtin_amdgcn_sched_barrier(0);
                    epi(sub, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (sub + 1 < NSUB) mm(sub + 1, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    epi(sub, 1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (sub + 1 < NSUB) mm(sub + 1, 1);
                    if (sub + 2 < NSUB) ldb(sub + 2);
                }
                // the next tile goes into the other buffer now, before this
                // tile's score stores are issued: waiting for its loads then
                // does not also wait for the stores
                if (more) stage(buf ^ 1);
                // QPW rows x 64 keys out of LDS: lane l takes 16 bytes of row
                // 4j + l/16 per step, each row a whole 256-byte segment
                const int c = lane & 15;
#pragma unroll
                for (int j = 0; j < QPW / 4; ++j) {
                    const int r = 4 * j + (lane >> 4);
                    const int t = tw0 + r;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(&ost[r * OST + 4 * c]);
                    if (!MASKED) {
                        __builtin_amdgcn_raw_buffer_store_b128(v, o_rs, o_voff[j], 4 * s0, 0);
                    } else if (t < T) {
                        if (vec_out) {
                            if (s0 + 4 * c < s_end) __builtin_amdgcn_raw_buffer_store_b128(v, o_rs, o_voff[j], 4 * s0, 0);
                        } else {
                            float* dst = out_b + (size_t)t * N + s0 + 4 * c;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (s0 + 4 * c + e < s_end) dst[e] = __builtin_bit_cast(float, v[e]);
                        }
                    }
                }
            } else if (more) {
                stage(buf ^ 1);
            }
            __syncthreads();
        };

        // leading tiles with every key visible to every query of the
        // workgroup, all inside [s_begin, s_end), full 16-byte row chunks
        int n_clean = 0;
        if (vec_out && t0 + TQB <= T) {
            const int lim = min(q_offset + t0 + 1, s_end);  // keys below lim are clean
            n_clean = lim > s_begin ? min(n_tiles, (lim - s_begin) / TILE) : 0;
        }
        fetch(s_begin);
        stage(0);
        __syncthreads();
        int it = 0;
        for (; it < n_clean; ++it) tile(it, std::false_type{});
        for (; it < n_tiles; ++it) tile(it, std::true_type{});
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
// query pair and 16 keys (the layout of indexer_math.h).  NP query pairs per
// workgroup.
//
// Each wave walks blocks of 16*SU consecutive keys (the four waves take
// turns); the scores of 64 consecutive keys are gathered across lanes into
// one 256-byte store per query.  Key loads are unconditional (addresses
// clamped into the visible range; values past it are never stored unmasked)
// and the next block's loads are issued before this block's stores.
//
// FILTER (the decode selection): instead of storing scores, every causal
// score whose key is at or above its row's threshold (seg::kTheta, from
// indexer_sample_threshold) is appended, with its token index, to an LDS
// list per query row; at the end each list goes to the row's candidate list
// in the segmented top-k workspace with one global atomic.  A row whose
// candidates exceed seg::kCap is flagged instead.  Rows with at most k
// candidates are skipped (their selection is all of them).
constexpr int FKPW = 1024;            // keys per workgroup when filtering

template <bool FILL, int NP, bool FILTER>
__global__ __launch_bounds__(NT) void indexer_fp8_stream(
    const uint8_t* __restrict__ q, const float* __restrict__ qs, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const float* __restrict__ w, float* __restrict__ scores,
    uint32_t* __restrict__ seg_ws, int T, int N, int q_offset, int keys_per_wg, int top_k) {
    constexpr int SQ = 2 * NP;
    __shared__ uint32_t c_key[FILTER ? SQ : 1][FILTER ? FKPW : 1];
    __shared__ int32_t c_idx[FILTER ? SQ : 1][FILTER ? FKPW : 1];
    __shared__ uint32_t c_cnt[SQ], c_base[SQ];
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

    i32x8 a[NP];
    float ws[NP][4];
    int tl[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) pair_operands(q, qs, w, row0, tq0 + 2 * p, T, lane, &a[p], ws[p], &tl[p]);
    // FILTER: per query row of the workgroup, the threshold key (rows that
    // select everything get ~0u: nothing passes)
    uint32_t theta[SQ];
    if (FILTER) {
        if (tid < SQ) c_cnt[tid] = 0u;
#pragma unroll
        for (int r = 0; r < SQ; ++r) {
            const int t = tq0 + r;
            const bool sel = t < T && (long long)min((long long)N, (long long)q_offset + t + 1) > top_k;
            theta[r] = sel ? seg_ws[(row0 + t) * seg::kRowWords + seg::kTheta] : ~0u;
        }
        __syncthreads();
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
                float v = pair_score(half_score(mfma_fp8(a[p], bf), ws[p]), kss[u]);
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
                    if (!FILTER) {
                        if (in && tq < t_end) out_b[(size_t)tq * N + key] = v;
                    } else {
                        const int r = 2 * p + qq;
                        const uint32_t fk = fkey(v);
                        const bool pass = in && key <= q_offset + tq && fk >= theta[r];
                        const uint64_t bal = __ballot(pass);
                        if (bal) {
                            uint32_t at = 0;
                            if (lane == 0) at = atomicAdd(&c_cnt[r], (uint32_t)__popcll(bal));
                            at = __builtin_amdgcn_readfirstlane(at);
                            const uint32_t pos = at + __builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                            if (pass) {
                                c_key[r][pos] = fk;
                                c_idx[r][pos] = key;
                            }
                        }
                    }
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
    if (FILTER) {
        __syncthreads();
        if (tid < t_end - tq0 && c_cnt[tid] > 0u) {
            uint32_t* wr = seg_ws + (row0 + tq0 + tid) * seg::kRowWords;
            const uint32_t at = atomicAdd(&wr[seg::kCtr + 1], c_cnt[tid]);
            if (at + c_cnt[tid] > (uint32_t)seg::kCap) wr[seg::kCtr + 2] = 1u;
            c_base[tid] = at;
        }
        __syncthreads();
        for (int r = 0; r < t_end - tq0; ++r) {
            const uint32_t n = c_cnt[r], at = c_base[r];
            if (n == 0u || at + n > (uint32_t)seg::kCap) continue;
            uint32_t* wr = seg_ws + (row0 + tq0 + r) * seg::kRowWords;
            for (int i = tid; i < (int)n; i += NT) {
                wr[seg::kCKey + at + i] = c_key[r][i];
                wr[seg::kCIdx + at + i] = (uint32_t)c_idx[r][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per-row threshold for the decode selection.  One 1024-thread workgroup per
// row with more than k candidates scores S = min(1024, n_cand) keys: all of
// them for rows of fewer than 1024, otherwise 64 blocks of 16 consecutive
// keys spread evenly over the row (block j starts at key
// floor(j (n_cand - 16) / 63); a block's 2 KiB of keys come in one piece,
// where 1024 single keys cost a memory round trip each), with the stream
// layout's arithmetic, and takes the key of its r-th largest sample score rounded
// down to 22 bits, r = mu + 6 sqrt(mu) + 8 with mu = S k / n_cand the
// expected number of samples among the row's top k.  Keys at or above it
// hold the row's top k unless the sample is far from typical, and the
// selection checks that (count >= k) before trusting it.  Also clears the
// row's candidate counter and overflow flag.
constexpr int SMP = 1024;
static_assert(SMP % 16 == 0, "the sample is whole 16-key blocks");
constexpr int SMT = TT;  // threads (the block helpers of topk_select.h assume TT)

__global__ __launch_bounds__(SMT) void indexer_sample_threshold(
    const uint8_t* __restrict__ q, const float* __restrict__ qs, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const float* __restrict__ w, uint32_t* __restrict__ seg_ws,
    int T, int N, int q_offset, int top_k) {
    __shared__ uint32_t skey[SMP];
    __shared__ uint32_t hist[seg::kBins];
    __shared__ uint32_t sh[SMT / 64 + 1];
    __shared__ uint32_t res[3];
    const size_t row = blockIdx.x;
    const int b = (int)(row / T), t = (int)(row % T);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, kb = lane >> 4;
    uint32_t* wr = seg_ws + row * seg::kRowWords;
    const int n_cand = (int)min((long long)N, (long long)q_offset + t + 1);
    if (tid == 0) {
        wr[seg::kCtr + 1] = 0u;
        wr[seg::kCtr + 2] = 0u;
    }
    if (n_cand <= top_k) return;
    const int S = min(SMP, n_cand);
    const uint8_t* __restrict__ k_b = k + (size_t)b * N * DI;
    const float* __restrict__ ks_b = ks + (size_t)b * N;
    i32x8 a;
    float ws4[4];
    int tl;
    pair_operands(q, qs, w, (size_t)b * T, t, t + 1, lane, &a, ws4, &tl);
    // 16 waves x 4 fragments of 16 samples
    constexpr int FPW = SMP / 16 / (SMT / 64);
    uint4 x0[FPW], x1[FPW];
    float kss[FPW];
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
        const int i = 16 * (FPW * wave + f) + m;
        const int s = S < SMP ? min(i, S - 1)
                              : (int)(((long long)(i >> 4) * (n_cand - 16)) / (SMP / 16 - 1)) + (i & 15);
        const uint4* p = reinterpret_cast<const uint4*>(k_b + (size_t)s * DI + 32 * kb);
        x0[f] = p[0];
        x1[f] = p[1];
        kss[f] = ks_b[s];
    }
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
        const float v = pair_score(half_score(mfma_fp8(a, pack8(x0[f], x1[f])), ws4), kss[f]);
        const int i = 16 * (FPW * wave + f) + m;
        if (kb == 0 && i < S) skey[i] = fkey(v);
    }
    __syncthreads();
    const uint32_t theta = sample_threshold(skey, S, top_k, n_cand, 6.f, 8.f, hist, sh, res);
    if (tid == 0) wr[seg::kTheta] = theta;
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
            DSA_TIMED("indexer_fp8_tiled<true>", stream,
                      indexer_fp8_tiled<true><<<grid, NTT, 0, stream>>>(q, qs, k, ks, w, scores, T, N,
                                                                        q_offset, (int)kpw));
        else
            DSA_TIMED("indexer_fp8_tiled<false>", stream,
                      indexer_fp8_tiled<false><<<grid, NTT, 0, stream>>>(q, qs, k, ks, w, scores, T, N,
                                                                         q_offset, (int)kpw));
        return launch_status();
    }
    const int np = T <= 2 ? 1 : 2;
    const int nqg = ceil_div(T, 2 * np);
    long long kpw = (long long)nqg * B * n_vis / DSA_STREAM_WG_TARGET;
    kpw = std::max<long long>(1024, std::min<long long>(16384, kpw));
    kpw = (kpw + 64 * SU - 1) / (64 * SU) * (64 * SU);
    dim3 grid(ceil_div(n_vis, kpw), nqg, B);
    auto go = [&](auto kern, const char* name) {
        DSA_TIMED(name, stream,
                  kern<<<grid, NT, 0, stream>>>(q, qs, k, ks, w, scores, nullptr, T, N, q_offset,
                                                (int)kpw, 0));
    };
    if (np == 1) {
        if (fill_masked) go(indexer_fp8_stream<true, 1, false>, "indexer_fp8_stream<true, 1, false>");
        else go(indexer_fp8_stream<false, 1, false>, "indexer_fp8_stream<false, 1, false>");
    } else {
        if (fill_masked) go(indexer_fp8_stream<true, 2, false>, "indexer_fp8_stream<true, 2, false>");
        else go(indexer_fp8_stream<false, 2, false>, "indexer_fp8_stream<false, 2, false>");
    }
    return launch_status();
}

bool indexer_filters(int B, int T) { return T < 16 && topk_segmented((long long)B * T); }

dsa_status launch_indexer_sample_threshold(const uint8_t* q, const float* qs, const uint8_t* k,
                                           const float* ks, const float* w, uint32_t* seg_ws,
                                           int B, int T, int N, int q_offset, int top_k,
                                           hipStream_t stream) {
    if (!indexer_filters(B, T)) return DSA_ERR_UNSUPPORTED;
    DSA_TIMED("indexer_sample_threshold", stream,
              indexer_sample_threshold<<<dim3((unsigned)(B * T)), SMT, 0, stream>>>(
                  q, qs, k, ks, w, seg_ws, T, N, q_offset, top_k));
    return launch_status();
}

dsa_status launch_indexer_fp8_filtered(const uint8_t* q, const float* qs, const uint8_t* k,
                                       const float* ks, const float* w, uint32_t* seg_ws,
                                       int B, int T, int N, int q_offset, int top_k,
                                       hipStream_t stream) {
    if (!indexer_filters(B, T)) return DSA_ERR_UNSUPPORTED;
    const long long n_vis = std::min<long long>(N, (long long)q_offset + T);
    const int np = T <= 2 ? 1 : 2;
    const int nqg = ceil_div(T, 2 * np);
    static_assert(FKPW % (64 * SU) == 0, "filtered key ranges are whole blocks");
    dim3 grid(ceil_div(n_vis, FKPW), nqg, B);
    auto go = [&](auto kern, const char* name) {
        DSA_TIMED(name, stream,
                  kern<<<grid, NT, 0, stream>>>(q, qs, k, ks, w, nullptr, seg_ws, T, N, q_offset, FKPW,
                                                top_k));
    };
    if (np == 1) go(indexer_fp8_stream<false, 1, true>, "indexer_fp8_stream<false, 1, true>");
    else go(indexer_fp8_stream<false, 2, true>, "indexer_fp8_stream<false, 2, true>");
    return launch_status();
}

dsa_status launch_indexer_f32(const float* q, const float* k, const float* w, float* scores,
                              int B, int T, int N, int H_I, int d_I, int q_offset,
                              bool fill_masked, hipStream_t stream) {
    if (H_I * d_I > F32_MAX_HD || H_I > 16) return DSA_ERR_UNSUPPORTED;
    dim3 grid(ceil_div(N, NT), T, B);
    DSA_TIMED("indexer_f32_kernel", stream,
              indexer_f32_kernel<<<grid, NT, 0, stream>>>(q, k, w, scores, T, N, H_I, d_I, q_offset,
                                                          fill_masked ? 1 : 0));
    return launch_status();
}

}  // namespace dsa
