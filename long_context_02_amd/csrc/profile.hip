// Per-kernel timing of the library's launches (a diagnostic, off by
// default).  While a profiling window is open, every launch site records a
// HIP event on its stream right before and right after the kernel; closing
// the window waits for those events and sums the elapsed times per kernel.
// Events are host-side objects created when the window opens; no device
// memory is allocated.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "dsa_internal.h"

namespace dsa {
namespace prof {
namespace {

struct Slot {
    const char* name;
    hipEvent_t start, stop;
    bool used;
};

std::mutex g_mu;                  // guards opening and closing a window
std::atomic<bool> g_on{false};
std::atomic<int> g_next{0};       // next free slot of the open window
std::vector<Slot> g_slots;

}  // namespace

bool enabled() { return g_on.load(std::memory_order_acquire); }

Scope::Scope(const char* name, hipStream_t s) : slot_(-1), stream_(s) {
    if (!enabled()) return;
    const int i = g_next.fetch_add(1, std::memory_order_relaxed);
    if (i >= (int)g_slots.size()) return;  // window full: not recorded
    g_slots[i].name = name;
    if (hipEventRecord(g_slots[i].start, s) != hipSuccess) return;
    slot_ = i;
}

Scope::~Scope() {
    if (slot_ < 0) return;
    if (hipEventRecord(g_slots[slot_].stop, stream_) == hipSuccess) g_slots[slot_].used = true;
}

dsa_status open_window(int max_launches) {
    if (max_launches < 1 || max_launches > (1 << 20)) return DSA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_on.load()) return DSA_ERR_INVALID_ARG;  // already open
    g_slots.assign((size_t)max_launches, Slot{nullptr, nullptr, nullptr, false});
    for (auto& s : g_slots) {
        if (hipEventCreate(&s.start) != hipSuccess || hipEventCreate(&s.stop) != hipSuccess) {
            for (auto& t : g_slots) {
                if (t.start) (void)hipEventDestroy(t.start);
                if (t.stop) (void)hipEventDestroy(t.stop);
            }
            g_slots.clear();
            return DSA_ERR_HIP;
        }
    }
    g_next.store(0);
    g_on.store(true, std::memory_order_release);
    return DSA_OK;
}

int close_window(dsa_kernel_time* out, int max_out, int* dropped) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_on.load()) return -1;
    g_on.store(false, std::memory_order_release);
    const int recorded = std::min(g_next.load(), (int)g_slots.size());
    if (dropped) *dropped = std::max(0, g_next.load() - (int)g_slots.size());
    int n = 0;
    bool ok = true;
    for (int i = 0; i < recorded; ++i) {
        Slot& s = g_slots[i];
        if (!s.used) continue;
        if (hipEventSynchronize(s.stop) != hipSuccess) {
            ok = false;
            continue;
        }
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, s.start, s.stop) != hipSuccess) {
            ok = false;
            continue;
        }
        int j = 0;
        while (j < n && out[j].name != s.name) ++j;
        if (j == n) {
            if (n == max_out) continue;  // more distinct kernels than entries
            out[n].name = s.name;
            out[n].launches = 0;
            out[n].total_ms = 0.0;
            ++n;
        }
        out[j].launches += 1;
        out[j].total_ms += ms;
    }
    for (auto& s : g_slots) {
        (void)hipEventDestroy(s.start);
        (void)hipEventDestroy(s.stop);
    }
    g_slots.clear();
    return ok ? n : -1;
}

// ---- peak probes ---------------------------------------------------------
namespace {
// A streaming read: every thread reads 16-byte pieces of the buffer in a
// grid-stride loop and adds their words; one value per workgroup is written
// so the loads cannot be dropped.
__global__ __launch_bounds__(256) void probe_stream_read(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) acc += p[i].x;
    acc += __shfl_xor(acc, 1, 64);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

// Back-to-back independent MFMAs (eight accumulators per wave, no memory
// traffic in the loop): the MFMA rate this chip sustains, at whatever engine
// clock it runs under that load.  FP8 = v_mfma_scale_f32_16x16x128_f8f6f4,
// otherwise v_mfma_f32_16x16x32_bf16.
typedef float f32x16 __attribute__((ext_vector_type(16)));

// The same with v_mfma_f32_32x32x16_bf16 (32768 FLOP each, four accumulators).
__global__ __launch_bounds__(256) void probe_mfma_32(int iters, float* __restrict__ sink) {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    const int l = (int)threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (l + e));
        b[e] = (__bf16)(0.002f * (l - e));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    if (s == 12345.f) sink[blockIdx.x] = s;
}

template <bool FP8>
__global__ __launch_bounds__(256) void probe_mfma(int iters, float* __restrict__ sink) {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int l = (int)threadIdx.x;
    if (FP8) {
        const i32x8 a = {l, l + 1, l + 2, l + 3, l + 4, l + 5, l + 6, l + 7};
        const i32x8 b = {l ^ 5, l ^ 6, l ^ 7, l ^ 8, l ^ 9, l ^ 10, l ^ 11, l ^ 12};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
    } else {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)(0.001f * (l + e));
            b[e] = (__bf16)(0.002f * (l - e));
        }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (s == 12345.f) sink[blockIdx.x] = s;  // keeps the loop; practically never stores
}

}  // namespace

}  // namespace prof
}  // namespace dsa

extern "C" {

double dsa_probe_peak(int what, const void* buf, size_t bytes, void* stream) {
    using namespace dsa::prof;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.0;
    double result = -1.0;
    const int reps = 5;
    float best = 0.f;
    if (what == DSA_PROBE_STREAM_READ) {
        if (!buf || bytes < (1u << 20) || ((uintptr_t)buf & 15u) != 0) goto done;
        const unsigned grid = 256u * 32u;
        // the buffer's first bytes - 64 KiB are read; the per-workgroup sums
        // go to its last 32 KiB
        const size_t n16 = (bytes - 65536) / 16;
        uint32_t* sink = reinterpret_cast<uint32_t*>(const_cast<char*>(static_cast<const char*>(buf)) +
                                                     (bytes - 32768) / 16 * 16);
        for (int r = 0; r < reps; ++r) {
            if (hipEventRecord(e0, s) != hipSuccess) goto done;
            probe_stream_read<<<grid, 256, 0, s>>>(static_cast<const uint4*>(buf), n16, sink);
            if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) goto done;
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) goto done;
            const float gbs = (float)(n16 * 16) / (ms * 1e-3f) / 1e9f;
            best = std::max(best, gbs);
        }
        result = best;
    } else if (what == DSA_PROBE_MFMA_BF16 || what == DSA_PROBE_MFMA_FP8 ||
               what == DSA_PROBE_MFMA_BF16_32X32) {
        const bool fp8 = what == DSA_PROBE_MFMA_FP8;
        const bool big = what == DSA_PROBE_MFMA_BF16_32X32;
        const int iters = 2048;
        const unsigned grid = 256u * 8u;  // 8 workgroups of 4 waves per CU
        float* sink = reinterpret_cast<float*>(const_cast<void*>(buf));
        if (!sink) goto done;
        for (int r = 0; r < reps; ++r) {
            if (hipEventRecord(e0, s) != hipSuccess) goto done;
            if (big) probe_mfma_32<<<grid, 256, 0, s>>>(iters, sink);
            else if (fp8) probe_mfma<true><<<grid, 256, 0, s>>>(iters, sink);
            else probe_mfma<false><<<grid, 256, 0, s>>>(iters, sink);
            if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) goto done;
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) goto done;
            const double flop = big ? (double)grid * 4 * iters * 4 * 32768.0
                                    : (double)grid * 4 * iters * 8 * (fp8 ? 65536.0 : 16384.0);
            best = std::max(best, (float)(flop / (ms * 1e-3) / 1e12));
        }
        result = best;
    }
done:
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return result;
}


dsa_status dsa_profile_start(int max_launches) { return dsa::prof::open_window(max_launches); }

int dsa_profile_stop(dsa_kernel_time* out, int max_out, int* dropped) {
    if ((!out && max_out > 0) || max_out < 0) return -1;
    return dsa::prof::close_window(out, max_out, dropped);
}

}  // extern "C"
