// Indexer alignment objective on gfx950 ("Paper Breakdown: DeepSeek-V3.2",
// section 2, "Continued Pre-Training (§2.1.1)"): the dense warm-up trains the
// indexer with L^I = sum_t KL(p_t || Softmax(I_t)), sparse training keeps the
// KL on the selected set S_t.  Per row, over the row's entries (the causal
// candidates s <= q_offset + t, or the valid selected slots):
//     lse  = log sum_s exp(I_s)
//     loss = sum_{p_s > 0} p_s (log p_s - (I_s - lse))
//     dL/dI_s = P exp(I_s - lse) - p_s,   P = sum_s p_s
// (the target is taken as given; for a distribution P = 1).
//
// Dense: one 1024-thread workgroup per row, two passes over the row.  Pass 1
// streams I and p once for the running max / exp-sum (lse) and P; pass 2
// streams them again for the loss terms and writes the gradient (zeros past
// the causal range).  HBM-bound: 16 B read and 4 B written per candidate.
// Sparse: one 256-thread workgroup per row gathers the k selected scores.
// Everything in fp32 with the library expf / logf.
#include <cmath>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int KT = 1024;   // dense: threads per row
constexpr int ST = 256;    // sparse: threads per row

struct Acc {
    float m;  // running max
    float l;  // sum exp(I - m)
};

__device__ __forceinline__ Acc acc_merge(Acc a, Acc b) {
    const float m = fmaxf(a.m, b.m);
    if (m == -__builtin_inff()) return Acc{m, 0.f};
    return Acc{m, a.l * expf(a.m - m) + b.l * expf(b.m - m)};
}

// add exp(x) to the running sum; x = -inf adds nothing (scores are finite
// or -inf)
__device__ __forceinline__ Acc acc_add(Acc a, float x) {
    if (x == -__builtin_inff()) return a;
    if (x <= a.m) return Acc{a.m, a.l + expf(x - a.m)};
    return Acc{x, a.l * expf(a.m - x) + 1.f};  // new max (from -inf: a.l = 0)
}

// Block-wide reductions (NTH threads, shared scratch of NTH/64 entries).
template <int NTH>
__device__ __forceinline__ Acc block_acc(Acc a, Acc* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        Acc o{__shfl_xor(a.m, off, 64), __shfl_xor(a.l, off, 64)};
        a = acc_merge(a, o);
    }
    __syncthreads();
    if (lane == 0) sh[w] = a;
    __syncthreads();
    Acc r = sh[0];
    for (int i = 1; i < NTH / 64; ++i) r = acc_merge(r, sh[i]);
    return r;
}

template <int NTH>
__device__ __forceinline__ float block_sum(float v, float* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    __syncthreads();
    if (lane == 0) sh[w] = v;
    __syncthreads();
    float r = 0.f;
    for (int i = 0; i < NTH / 64; ++i) r += sh[i];
    return r;
}

__device__ __forceinline__ float kl_term(float pv, float d) {  // p (log p - d), 0 for p = 0
    return pv > 0.f ? pv * (logf(pv) - d) : 0.f;
}

// four consecutive entries at once; entries equal to -inf add nothing
__device__ __forceinline__ Acc acc_add4(Acc a, const float4& x) {
    const float m4 = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
    if (m4 == -__builtin_inff()) return a;
    if (m4 > a.m) {
        a.l *= expf(a.m - m4);  // from -inf: a.l = 0
        a.m = m4;
    }
    a.l += expf(x.x - a.m) + expf(x.y - a.m) + expf(x.z - a.m) + expf(x.w - a.m);
    return a;
}

__global__ __launch_bounds__(KT) void indexer_kl_dense(const float* __restrict__ scores,
                                                       const float* __restrict__ p,
                                                       float* __restrict__ loss, float* __restrict__ grad,
                                                       int T, int N, int q_offset) {
    __shared__ Acc sh_acc[KT / 64];
    __shared__ float sh_f[KT / 64];
    const size_t row = blockIdx.x;
    const int t = (int)(row % (size_t)T);
    const int n = (int)min((long long)N, (long long)q_offset + t + 1);
    const float* __restrict__ I = scores + row * N;
    const float* __restrict__ pr = p + row * N;
    float* __restrict__ gr = grad ? grad + row * N : nullptr;
    // rows of a multiple of 4 entries are 16-byte aligned: whole float4s over
    // [0, 4*n4), single entries over the rest
    const bool vec = (N & 3) == 0;
    const int n4 = vec ? n >> 2 : 0;

    Acc a{-__builtin_inff(), 0.f};
    float P = 0.f;
#pragma unroll 2
    for (int j = threadIdx.x; j < n4; j += KT) {
        const float4 x = reinterpret_cast<const float4*>(I)[j];
        const float4 pv = reinterpret_cast<const float4*>(pr)[j];
        a = acc_add4(a, x);
        P += (pv.x + pv.y) + (pv.z + pv.w);
    }
    for (int s = 4 * n4 + threadIdx.x; s < n; s += KT) {
        a = acc_add(a, I[s]);
        P += pr[s];
    }
    a = block_acc<KT>(a, sh_acc);
    P = block_sum<KT>(P, sh_f);
    const float lse = a.m + logf(a.l);

    float L = 0.f;
#pragma unroll 2
    for (int j = threadIdx.x; j < n4; j += KT) {
        const float4 x = reinterpret_cast<const float4*>(I)[j];
        const float4 pv = reinterpret_cast<const float4*>(pr)[j];
        const float4 d = {x.x - lse, x.y - lse, x.z - lse, x.w - lse};
        L += (kl_term(pv.x, d.x) + kl_term(pv.y, d.y)) + (kl_term(pv.z, d.z) + kl_term(pv.w, d.w));
        if (gr)
            reinterpret_cast<float4*>(gr)[j] =
                float4{P * expf(d.x) - pv.x, P * expf(d.y) - pv.y, P * expf(d.z) - pv.z, P * expf(d.w) - pv.w};
    }
    for (int s = 4 * n4 + threadIdx.x; s < n; s += KT) {
        const float d = I[s] - lse;
        const float pv = pr[s];
        L += kl_term(pv, d);
        if (gr) gr[s] = P * expf(d) - pv;
    }
    if (gr) {  // zeros past the causal range
        const int z0 = (n + 3) & ~3;
        for (int s = n + threadIdx.x; s < min(z0, N); s += KT) gr[s] = 0.f;
        if (vec)
            for (int j = (z0 >> 2) + threadIdx.x; j < (N >> 2); j += KT)
                reinterpret_cast<float4*>(gr)[j] = float4{0.f, 0.f, 0.f, 0.f};
        else
            for (int s = z0 + threadIdx.x; s < N; s += KT) gr[s] = 0.f;
    }
    L = block_sum<KT>(L, sh_f);
    if (threadIdx.x == 0) loss[row] = L;
}

__global__ __launch_bounds__(ST) void indexer_kl_sparse(const float* __restrict__ scores,
                                                        const float* __restrict__ p_sel,
                                                        const int32_t* __restrict__ idx,
                                                        float* __restrict__ loss,
                                                        float* __restrict__ grad, int N, int k) {
    __shared__ Acc sh_acc[ST / 64];
    __shared__ float sh_f[ST / 64];
    constexpr int PER = 8;  // slots per thread and round (k <= 2048 = ST * PER)
    const size_t row = blockIdx.x;
    const float* __restrict__ I = scores + row * N;
    const int32_t* __restrict__ ir = idx + row * k;
    const float* __restrict__ pr = p_sel + row * k;

    // every slot this thread owns: index, target and score, loads issued together
    float xs[PER], ps[PER];
    bool ok[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i = threadIdx.x + u * ST;
        const int s = i < k ? ir[i] : -1;
        ok[u] = s >= 0 && s < N;
        ps[u] = ok[u] ? pr[i] : 0.f;
        xs[u] = ok[u] ? I[s] : -__builtin_inff();
    }
    Acc a{-__builtin_inff(), 0.f};
    float P = 0.f;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        a = acc_add(a, xs[u]);
        P += ps[u];
    }
    a = block_acc<ST>(a, sh_acc);
    P = block_sum<ST>(P, sh_f);
    const float lse = a.m + logf(a.l);

    float L = 0.f;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i = threadIdx.x + u * ST;
        float g = 0.f;
        if (ok[u]) {
            const float d = xs[u] - lse;
            L += kl_term(ps[u], d);
            g = P * expf(d) - ps[u];
        }
        if (grad && i < k) grad[row * k + i] = g;
    }
    L = block_sum<ST>(L, sh_f);
    if (threadIdx.x == 0) loss[row] = L;
}

}  // namespace

dsa_status launch_indexer_kl(const float* scores, const float* p, const int32_t* idx, float* loss,
                             float* grad, int B, int T, int N, int k, int q_offset, hipStream_t stream) {
    const unsigned rows = (unsigned)((long long)B * T);
    if (idx == nullptr)
        DSA_TIMED("indexer_kl_dense", stream,
                  indexer_kl_dense<<<rows, KT, 0, stream>>>(scores, p, loss, grad, T, N, q_offset));
    else
        DSA_TIMED("indexer_kl_sparse", stream,
                  indexer_kl_sparse<<<rows, ST, 0, stream>>>(scores, p, idx, loss, grad, N, k));
    return launch_status();
}

}  // namespace dsa
