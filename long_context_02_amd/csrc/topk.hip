// Per-query causal top-k token selection on gfx950.
//
// Selection ("Paper Breakdown: DeepSeek-V3.2", section 2 "Architecture: DSA
// (§2.1)"): query t keeps the k tokens with the largest index scores among
// its causal candidates s < min(N, q_offset + t + 1).  Ties go to the lower
// index, -0 equals +0, NaN ranks lowest; the kept indices are written in
// ascending order and padded with -1.
//
// One 1024-thread workgroup per row, radix select on an order-preserving
// 32-bit key:
//   pass 1 (HBM)  LDS histogram of the top 12 key bits -> the bin b1 holding
//                 the k-th largest key, the count above it and in it;
//   pass 2 (HBM)  ordered compaction: keys above b1 go to list A (they are
//                 kept for sure), keys inside b1 go to an LDS candidate list
//                 C with their indices, both in index order (a block-wide
//                 exclusive scan over per-thread counts built from
//                 wave-level prefix sums);
//   in LDS        two more 10-bit digits over C give the exact k-th key K*
//                 and how many of the keys equal to K* to keep; an ordered
//                 scan over C keeps every key > K* and the lowest-index keys
//                 == K* (list B);
//   merge         A and B are both ascending; each element's output slot is
//                 its rank in its own list plus its rank in the other.
// When bin b1 holds more keys than the LDS list can take (e.g. a row of
// identical scores) the remaining digits are resolved with further HBM
// passes and a final ordered emission pass over the row.
//
// Batches of few rows (decode: one row per sequence) instead split every row
// over several workgroups; see the segmented path below.
#include "indexer_math.h"
#include "topk_select.h"

namespace dsa {
namespace {

// One pass per row.  A threshold from a sample of the row (128 blocks of 16
// consecutive scores spread over it) filters the keys while the row is read
// once; each wave appends the keys at or above it to its own LDS region
// (positions from a ballot, no atomics), the waves taking interleaved 64-key
// blocks so that a dense stretch of high scores spreads over all of them.
// The exact top-k is then selected among the candidates (all CAP1 slots; the
// unused ones hold key 0).  A row whose sample
// misleads (fewer than k candidates, or a wave region full) and short rows
// take the two-pass selection instead.
constexpr int SAMP_BLOCKS = 128, SAMP_BLK = 16, SAMP = SAMP_BLOCKS * SAMP_BLK;
constexpr int WREG = 384;              // candidate slots per wave
constexpr int CAP1 = WREG * NW;        // 6144
constexpr int ONEPASS_LDS_WORDS = 2 * CAP1 + BINS + NW + 1 + 3 + NW + 1;
constexpr int ROWS_LDS_WORDS = ONEPASS_LDS_WORDS > ROW_LDS_WORDS ? ONEPASS_LDS_WORDS : ROW_LDS_WORDS;

__global__ __launch_bounds__(TT) void topk_rows(const float* __restrict__ scores,
                                                int32_t* __restrict__ idx, int T, int N, int k,
                                                int q_offset) {
    __shared__ uint32_t lds[ROWS_LDS_WORDS];
    const int t = blockIdx.x, b = blockIdx.y;
    const size_t row = (size_t)b * T + t;
    const int n_cand = (int)min((long long)N, (long long)q_offset + t + 1);
    int32_t* __restrict__ out = idx + row * k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n_cand <= k) {  // every candidate is kept
        for (int i = tid; i < k; i += TT) out[i] = i < n_cand ? i : -1;
        return;
    }
    const float* __restrict__ s = scores + row * N;
    if (n_cand < 16 * SAMP) {  // shorter rows: the two-pass selection is faster
        select_row(s, out, n_cand, k, carve_row_lds(lds));
        return;
    }
    uint32_t* ckey = lds;                                        // CAP1 (first the sample)
    int32_t* cidx = reinterpret_cast<int32_t*>(lds + CAP1);      // CAP1
    uint32_t* hist = lds + 2 * CAP1;                             // BINS
    uint32_t* sh = hist + BINS;                                  // NW + 1
    uint32_t* res = sh + NW + 1;                                 // 3
    uint32_t* wcnt = res + 3;                                    // NW + 1
    // sample: block j starts at j * (n_cand - 16) / 127; 8 threads x 2 keys per block
    {
        const int j = tid >> 3, o = 2 * (tid & 7);
        const int st = (int)(((long long)j * (n_cand - SAMP_BLK)) / (SAMP_BLOCKS - 1));
        ckey[SAMP_BLK * j + o] = fkey(s[st + o]);
        ckey[SAMP_BLK * j + o + 1] = fkey(s[st + o + 1]);
    }
    __syncthreads();
    const uint32_t theta = sample_threshold(ckey, SAMP, k, n_cand, 4.f, 4.f, hist, sh, res);
    // one pass: lane l of wave w reads 4 scores of 64-key block 16*(l/16) + w
    // of each 4096-key stretch, at offset 4*(l%16)
    const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15u) == 0);
    uint32_t* wkey = ckey + WREG * wave;
    int32_t* widx = cidx + WREG * wave;
    uint32_t fill = 0;  // wave-uniform
    // RU stretches per round: their loads are all in flight before the first
    // is filtered (the row is read once, so the read rate is set by the
    // bytes in flight per CU)
    constexpr int RU = 4;
    for (int base0 = 0; base0 < n_cand; base0 += 4 * TT * RU) {
        float v[RU][4];
#pragma unroll
        for (int u = 0; u < RU; ++u)
            load4(s, base0 + 4 * TT * u + 64 * (16 * (lane >> 4) + wave) + 4 * (lane & 15), n_cand, vec,
                  v[u]);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int e = base0 + 4 * TT * u + 64 * (16 * (lane >> 4) + wave) + 4 * (lane & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = fkey(v[u][j]);
                const bool pass = e + j < n_cand && key >= theta;
                const uint64_t bal = __ballot(pass);
                const uint32_t c = (uint32_t)__popcll(bal);
                if (c == 0u) continue;
                const uint32_t pos = fill + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (pass && pos < (uint32_t)WREG) {
                    wkey[pos] = key;
                    widx[pos] = e + j;
                }
                fill += c;
            }
        }
    }
    // the wave's unused slots get key 0, below the (positive) threshold: never
    // picked, never tied with the k-th key
    for (int i = (int)fill + lane; i < WREG; i += 64) wkey[i] = 0u;
    if (lane == 0) wcnt[wave] = fill;
    __syncthreads();
    uint32_t n_c = 0;
    bool over = false;
    for (int w = 0; w < NW; ++w) {
        const uint32_t c = wcnt[w];
        over |= c > (uint32_t)WREG;
        n_c += c;
    }
    if (over || n_c < (uint32_t)k) {
        __syncthreads();
        select_row(s, out, n_cand, k, carve_row_lds(lds));
        return;
    }
    select_candidates<TT, true>(ckey, cidx, CAP1, k, n_cand, out, hist, sh, res);
}

// ---------------------------------------------------------------------------
// Segmented selection for batches of few long rows (decode): every row is
// split into SEG-element segments handled by separate workgroups.
//   topk_seg_zero      clear each row's histogram and counters
//   topk_seg_hist      LDS histogram of the top 12 key bits of a segment,
//                      added into the row's histogram in the workspace
//   topk_seg_collect   from the row histogram: the bin b1 of the k-th largest
//                      key; keys above b1 are appended to the row's list of
//                      sure picks, keys in b1 (with their index) to its
//                      candidate list (one atomic per list and workgroup)
//   topk_seg_finalize  per row: the exact k-th key among the candidates, the
//                      lowest-index ties, and the k picks written in ascending
//                      order through an index bitmap; a row whose b1 holds
//                      more than CAPG keys is selected by the single-workgroup
//                      path instead
constexpr int SEG = 16384;              // elements per segment
constexpr int STT = TT;                 // threads of the segment kernels
constexpr int CAPG = seg::kCap;         // candidate capacity per row
// per-row workspace, in 32-bit words
constexpr int WS_HIST = seg::kHist, WS_CTR = seg::kCtr, WS_DEF = seg::kDef, WS_CKEY = seg::kCKey,
              WS_CIDX = seg::kCIdx, WS_ROW = seg::kRowWords;
// counters: [0] sure picks, [1] candidates, [2] candidate overflow flag

__device__ __forceinline__ int row_candidates(int t, int N, int q_offset) {
    return (int)min((long long)N, (long long)q_offset + t + 1);
}

__global__ __launch_bounds__(STT) void topk_seg_zero(uint32_t* __restrict__ ws) {
    uint32_t* w = ws + (size_t)blockIdx.x * WS_ROW;
    for (int i = threadIdx.x; i < WS_DEF; i += STT) w[i] = 0u;
}

__global__ __launch_bounds__(STT) void topk_seg_hist(const float* __restrict__ scores,
                                                     uint32_t* __restrict__ ws, int T, int N, int k,
                                                     int q_offset) {
    __shared__ uint32_t hist[BINS];
    const int row = blockIdx.y, t = row % T;
    const int n_cand = row_candidates(t, N, q_offset);
    const int s0 = blockIdx.x * SEG, s1 = min(n_cand, s0 + SEG);
    if (n_cand <= k || s0 >= s1) return;
    const float* __restrict__ s = scores + (size_t)row * N;
    const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15u) == 0);
    for (int i = threadIdx.x; i < BINS; i += STT) hist[i] = 0u;
    __syncthreads();
    constexpr int PER = SEG / (4 * STT);  // 4-key groups per thread
    float v[PER][4];
#pragma unroll
    for (int i = 0; i < PER; ++i) load4(s, s0 + 4 * (int)threadIdx.x + 4 * STT * i, s1, vec, v[i]);
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (s0 + 4 * (int)threadIdx.x + 4 * STT * i + j < s1) atomicAdd(&hist[fkey(v[i][j]) >> 20], 1u);
    __syncthreads();
    uint32_t* gh = ws + (size_t)row * WS_ROW + WS_HIST;
    for (int i = threadIdx.x; i < BINS; i += STT)
        if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

__global__ __launch_bounds__(STT) void topk_seg_collect(const float* __restrict__ scores,
                                                        uint32_t* __restrict__ ws, int T, int N, int k,
                                                        int q_offset) {
    constexpr int PER = SEG / (4 * STT);  // 4-key groups per thread
    __shared__ uint4 kst[SEG / 4];        // the segment's keys; each thread reads back only its own
    __shared__ uint32_t hist[BINS];
    __shared__ uint32_t sh[NW + 1];
    __shared__ uint32_t res[3];
    __shared__ uint32_t base[2];
    const int row = blockIdx.y, t = row % T;
    const int n_cand = row_candidates(t, N, q_offset);
    const int s0 = blockIdx.x * SEG, s1 = min(n_cand, s0 + SEG);
    if (n_cand <= k || s0 >= s1) return;
    uint32_t* w = ws + (size_t)row * WS_ROW;
    const float* __restrict__ s = scores + (size_t)row * N;
    const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15u) == 0);
    const int tid = threadIdx.x;
    // out-of-range slots (last segment only) get key 0, in bin 0
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = s0 + 4 * tid + 4 * STT * i;
        float v[4];
        load4(s, e, s1, vec, v);
        kst[tid + STT * i] = make_uint4(fkey(v[0]), e + 1 < s1 ? fkey(v[1]) : 0u,
                                        e + 2 < s1 ? fkey(v[2]) : 0u, e + 3 < s1 ? fkey(v[3]) : 0u);
        if (e >= s1) kst[tid + STT * i].x = 0u;
    }
    {
        constexpr int HPT = BINS / STT;
        uint32_t hv[HPT];
#pragma unroll
        for (int j = 0; j < HPT; ++j) hv[j] = w[WS_HIST + tid + j * STT];
#pragma unroll
        for (int j = 0; j < HPT; ++j) hist[tid + j * STT] = hv[j];
    }
    __syncthreads();
    find_bin(hist, BINS, (uint32_t)k, sh, res);
    const uint32_t b1 = res[0], eq1 = res[2];
    if (eq1 > (uint32_t)CAPG) {  // the row takes the single-workgroup path
        if (blockIdx.x == 0 && tid == 0) w[WS_CTR + 2] = 1u;
        return;
    }
    // bin 0 slots past s1 are never above b1; they are skipped as candidates
    // when b1 is 0
    const int lim = (b1 == 0u) ? s1 : s0 + SEG;
    uint32_t nd = 0, nc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint4 q = kst[tid + STT * i];
        const int e = s0 + 4 * tid + 4 * STT * i;
        const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            nd += (kk[j] >> 20) > b1;
            nc += (kk[j] >> 20) == b1 && e + j < lim;
        }
    }
    // one scan of both counts (each below 2^16), one atomic per list
    uint32_t tot;
    const uint32_t pos = block_excl_scan((nd << 16) | nc, sh, &tot);
    if (tid == 0) {
        base[0] = (tot >> 16) ? atomicAdd(&w[WS_CTR + 0], tot >> 16) : 0u;
        base[1] = (tot & 0xFFFFu) ? atomicAdd(&w[WS_CTR + 1], tot & 0xFFFFu) : 0u;
    }
    __syncthreads();
    uint32_t pd = base[0] + (pos >> 16), pc = base[1] + (pos & 0xFFFFu);
    int32_t* def = reinterpret_cast<int32_t*>(w + WS_DEF);
    uint32_t* ckey = w + WS_CKEY;
    int32_t* cidx = reinterpret_cast<int32_t*>(w + WS_CIDX);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint4 q = kst[tid + STT * i];
        const int e = s0 + 4 * tid + 4 * STT * i;
        const uint32_t kk[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t bin = kk[j] >> 20;
            if (bin > b1) def[pd++] = e + j;
            else if (bin == b1 && e + j < lim) {
                ckey[pc] = kk[j];
                cidx[pc++] = e + j;
            }
        }
    }
}

// A row's candidate list (n_c <= CAPG keys and token indices) from its
// workspace into LDS; every load is issued before the first is waited for
// (a loop that stores each entry as it arrives waits for one memory round
// trip per iteration).
__device__ __forceinline__ void load_candidates(const uint32_t* __restrict__ wr, int n_c, uint32_t* ckey,
                                                int32_t* cidx) {
    constexpr int PER = (CAPG + TT - 1) / TT;
    const int tid = threadIdx.x;
    uint32_t kr[PER], ir[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + j * TT;
        kr[j] = i < n_c ? wr[WS_CKEY + i] : 0u;
        ir[j] = i < n_c ? wr[WS_CIDX + i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + j * TT;
        if (i < n_c) {
            ckey[i] = kr[j];
            cidx[i] = (int32_t)ir[j];
        }
    }
}

constexpr int FIN_LDS_WORDS = 2 * CAPG + BINS + NW + 1 + 3;
constexpr int K3_LDS_WORDS = FIN_LDS_WORDS > ROW_LDS_WORDS ? FIN_LDS_WORDS : ROW_LDS_WORDS;

__global__ __launch_bounds__(TT) void topk_seg_finalize(const float* __restrict__ scores,
                                                        const uint32_t* __restrict__ ws,
                                                        int32_t* __restrict__ idx, int T, int N, int k,
                                                        int q_offset) {
    __shared__ uint32_t lds[K3_LDS_WORDS];
    const int row = blockIdx.x, t = row % T;
    const int tid = threadIdx.x;
    const int n_cand = row_candidates(t, N, q_offset);
    int32_t* __restrict__ out = idx + (size_t)row * k;
    if (n_cand <= k) {
        for (int i = tid; i < k; i += TT) out[i] = i < n_cand ? i : -1;
        return;
    }
    const uint32_t* w = ws + (size_t)row * WS_ROW;
    if (w[WS_CTR + 2]) {
        select_row(scores + (size_t)row * N, out, n_cand, k, carve_row_lds(lds));
        return;
    }
    uint32_t* ckey = lds;                                     // CAPG
    int32_t* cidx = reinterpret_cast<int32_t*>(ckey + CAPG);  // CAPG
    uint32_t* hist = reinterpret_cast<uint32_t*>(cidx + CAPG);  // BINS, later the bitmap
    uint32_t* sh = hist + BINS;                               // NW + 1
    uint32_t* res = sh + NW + 1;                              // 3
    const int n_def = (int)w[WS_CTR + 0], n_c = (int)w[WS_CTR + 1];
    const int32_t* gdef = reinterpret_cast<const int32_t*>(w + WS_DEF);
    load_candidates(w, n_c, ckey, cidx);
    const uint32_t r1 = (uint32_t)(k - n_def);  // picks still to make among the candidates
    // digits 2 and 3 (key bits 19..10 and 9..0) give the exact k-th key
    for (int i = tid; i < 1024; i += TT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n_c; i += TT) atomicAdd(&hist[(ckey[i] >> 10) & 1023u], 1u);
    __syncthreads();
    find_bin(hist, 1024, r1, sh, res);
    const uint32_t b2 = res[0], r2 = r1 - res[1];
    for (int i = tid; i < 1024; i += TT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n_c; i += TT)
        if (((ckey[i] >> 10) & 1023u) == b2) atomicAdd(&hist[ckey[i] & 1023u], 1u);
    __syncthreads();
    find_bin(hist, 1024, r2, sh, res);
    const uint32_t b3 = res[0], n_tie = res[2];
    const uint32_t kthr = (ckey[0] & 0xFFF00000u) | (b2 << 10) | b3;  // the k-th key (bin b1 is shared)
    const uint32_t r3 = r2 - res[1];  // ties to keep, lowest indices first
    const uint32_t inv_thr = tie_threshold(ckey, cidx, n_c, kthr, n_tie, r3, hist, sh, res);
    emit_ascending(gdef, n_def, ckey, cidx, n_c, kthr, inv_thr, n_cand, out, hist, sh);
}


// ---------------------------------------------------------------------------
// Decode selection from candidate lists (built by the filtered indexer from
// a sampled threshold): one 1024-thread workgroup per row finds the exact
// k-th key among the row's candidates with the three radix digits, keeps the
// lowest-index ties and writes the picks in ascending order.  When the list
// holds fewer than k keys (the threshold was too high) or overflowed, the
// workgroup rescores the whole row into `scores`, with the stream layout's
// arithmetic (so the scores are those dsa_indexer_scores returns), and
// selects from there.
__device__ void rescore_row(const uint8_t* __restrict__ q, const float* __restrict__ qs,
                            const uint8_t* __restrict__ kk, const float* __restrict__ ks,
                            const float* __restrict__ w, float* __restrict__ srow, int b, int t,
                            int T, int N, int n_cand) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, kb = lane >> 4;
    const uint8_t* __restrict__ k_b = kk + (size_t)b * N * DI;
    const float* __restrict__ ks_b = ks + (size_t)b * N;
    i32x8 a;
    float ws4[4];
    int tl;
    pair_operands(q, qs, w, (size_t)b * T, t, t + 1, lane, &a, ws4, &tl);
    constexpr int U = 4;  // fragments in flight per wave
    for (int f0 = 16 * U * wave; f0 < n_cand; f0 += 16 * U * NW) {
        uint4 x0[U], x1[U];
        float kss[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = min(f0 + 16 * u + m, n_cand - 1);
            const uint4* p = reinterpret_cast<const uint4*>(k_b + (size_t)s * DI + 32 * kb);
            x0[u] = p[0];
            x1[u] = p[1];
            kss[u] = ks_b[s];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float v = pair_score(half_score(mfma_fp8(a, pack8(x0[u], x1[u])), ws4), kss[u]);
            const int s = f0 + 16 * u + m;
            if (kb == 0 && s < n_cand) srow[s] = v;
        }
    }
}

__global__ __launch_bounds__(TT) void topk_cand_select(
    const uint8_t* __restrict__ q, const float* __restrict__ qs, const uint8_t* __restrict__ kk,
    const float* __restrict__ ks, const float* __restrict__ w, float* __restrict__ scores,
    const uint32_t* __restrict__ ws, int32_t* __restrict__ idx, int T, int N, int k, int q_offset) {
    __shared__ uint32_t lds[K3_LDS_WORDS];
    const int row = blockIdx.x, t = row % T, b = row / T;
    const int tid = threadIdx.x;
    const int n_cand = row_candidates(t, N, q_offset);
    int32_t* __restrict__ out = idx + (size_t)row * k;
    if (n_cand <= k) {
        for (int i = tid; i < k; i += TT) out[i] = i < n_cand ? i : -1;
        return;
    }
    const uint32_t* wr = ws + (size_t)row * WS_ROW;
    const int n_c = (int)wr[WS_CTR + 1];
    if (wr[WS_CTR + 2] || n_c < k) {
        float* srow = scores + (size_t)row * N;
        rescore_row(q, qs, kk, ks, w, srow, b, t, T, N, n_cand);
        __threadfence();
        __syncthreads();
        select_row(srow, out, n_cand, k, carve_row_lds(lds));
        return;
    }
    uint32_t* ckey = lds;                                        // CAPG
    int32_t* cidx = reinterpret_cast<int32_t*>(ckey + CAPG);     // CAPG
    uint32_t* hist = reinterpret_cast<uint32_t*>(cidx + CAPG);   // BINS, later the bitmap
    uint32_t* sh = hist + BINS;                                  // NW + 1
    uint32_t* res = sh + NW + 1;                                 // 3
    load_candidates(wr, n_c, ckey, cidx);
    __syncthreads();
    select_candidates(ckey, cidx, n_c, k, n_cand, out, hist, sh, res);
}

}  // namespace

size_t topk_workspace_bytes(int B, int T, int, int) {
    const long long rows = (long long)B * T;
    return topk_segmented(rows) ? (size_t)rows * WS_ROW * sizeof(uint32_t) : 0;
}

dsa_status launch_topk(const float* scores, int32_t* idx, int B, int T, int N, int k,
                       int q_offset, void* workspace, hipStream_t stream) {
    if (k > KMAX) return DSA_ERR_UNSUPPORTED;
    if (B > 65535) return DSA_ERR_UNSUPPORTED;
    const long long rows = (long long)B * T;
    if (!topk_segmented(rows)) {
        topk_rows<<<dim3(T, B), TT, 0, stream>>>(scores, idx, T, N, k, q_offset);
        return launch_status();
    }
    // few long rows: several workgroups per row
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    const long long n_max = std::min<long long>(N, (long long)q_offset + T);
    const int nseg = (int)((n_max + SEG - 1) / SEG);
    topk_seg_zero<<<dim3((unsigned)rows), STT, 0, stream>>>(ws);
    topk_seg_hist<<<dim3(nseg, (unsigned)rows), STT, 0, stream>>>(scores, ws, T, N, k, q_offset);
    topk_seg_collect<<<dim3(nseg, (unsigned)rows), STT, 0, stream>>>(scores, ws, T, N, k, q_offset);
    topk_seg_finalize<<<dim3((unsigned)rows), TT, 0, stream>>>(scores, ws, idx, T, N, k, q_offset);
    return launch_status();
}

dsa_status launch_topk_from_candidates(const uint8_t* q, const float* qs, const uint8_t* kk,
                                       const float* ks, const float* w, float* scores,
                                       int32_t* idx, int B, int T, int N, int top_k, int q_offset,
                                       void* workspace, hipStream_t stream) {
    if (top_k > KMAX || !topk_segmented((long long)B * T)) return DSA_ERR_UNSUPPORTED;
    topk_cand_select<<<dim3((unsigned)(B * T)), TT, 0, stream>>>(
        q, qs, kk, ks, w, scores, static_cast<const uint32_t*>(workspace), idx, T, N, top_k, q_offset);
    return launch_status();
}

}  // namespace dsa
