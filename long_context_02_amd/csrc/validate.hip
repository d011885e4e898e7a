// Debug validation of caller-provided indices (environment DSA_VALIDATE=1).
//
// Entry points that take token indices or cache positions from the caller
// normally skip out-of-range entries.  In validation mode they first count,
// on the stream, the entries that are neither -1 nor inside [0, N) (token
// indices) or whose row pos[b] + t falls outside [0, N) (cache positions),
// wait for the stream, and refuse the call with DSA_ERR_BAD_INDEX when the
// count is not zero.  The count lives in one device word of the library;
// validated calls that overlap on one device share it.
#include <cstdlib>
#include <cstring>

#include "dsa_internal.h"

namespace dsa {
namespace {

__device__ unsigned int bad_count;

__global__ void clear_bad_count() {
    if (blockIdx.x == 0 && threadIdx.x == 0) bad_count = 0u;
}

__global__ __launch_bounds__(256) void count_bad_indices(const int32_t* __restrict__ idx, size_t n, int N) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    unsigned int bad = 0u;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int v = idx[i];
        bad += (v != -1 && (unsigned)v >= (unsigned)N) ? 1u : 0u;
    }
    if (bad) atomicAdd(&bad_count, bad);
}

__global__ __launch_bounds__(256) void count_bad_positions(const int32_t* __restrict__ pos, int B, int T,
                                                          int N) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const long long p0 = pos[b], p1 = p0 + T - 1;
    if (p0 < 0 || p1 >= N) atomicAdd(&bad_count, 1u);
}

// the count of the kernels just launched on s (waits for the stream)
dsa_status read_bad_count(hipStream_t s) {
    if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
    unsigned int host = 0u;
    if (hipMemcpyFromSymbolAsync(&host, HIP_SYMBOL(bad_count), sizeof(host), 0, hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return DSA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return DSA_ERR_HIP;
    return host == 0u ? DSA_OK : DSA_ERR_BAD_INDEX;
}

}  // namespace

bool validation_enabled() {
    const char* e = std::getenv("DSA_VALIDATE");
    return e != nullptr && std::strcmp(e, "1") == 0;
}

dsa_status validate_indices(const int32_t* idx, size_t n, int N, hipStream_t s) {
    clear_bad_count<<<1, 64, 0, s>>>();
    if (n > 0) {
        const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
        count_bad_indices<<<grid, 256, 0, s>>>(idx, n, N);
    }
    return read_bad_count(s);
}

dsa_status validate_positions(const int32_t* pos, int B, int T, int N, hipStream_t s) {
    clear_bad_count<<<1, 64, 0, s>>>();
    count_bad_positions<<<(unsigned)((B + 255) / 256), 256, 0, s>>>(pos, B, T, N);
    return read_bad_count(s);
}

}  // namespace dsa
