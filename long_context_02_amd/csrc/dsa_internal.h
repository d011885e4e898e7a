// Internal declarations shared by the libdsa translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workspace carving: every block starts on a 256-byte boundary.
inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// ---- indexer (indexer.hip) ------------------------------------------------
// fill_masked: write -inf over the non-causal part of every row (the public
// entry point promises that); the fused path skips those stores.
dsa_status launch_indexer_fp8(const uint8_t* q, const float* qs, const uint8_t* k,
                              const float* ks, const float* w, float* scores,
                              int B, int T, int N, int q_offset, bool fill_masked,
                              hipStream_t stream);
dsa_status launch_indexer_f32(const float* q, const float* k, const float* w, float* scores,
                              int B, int T, int N, int H_I, int d_I, int q_offset,
                              bool fill_masked, hipStream_t stream);

// ---- top-k (topk.hip) -----------------------------------------------------
size_t topk_workspace_bytes(int B, int T, int N, int k);
dsa_status launch_topk(const float* scores, int32_t* idx, int B, int T, int N, int k,
                       int q_offset, void* workspace, hipStream_t stream);

// ---- sparse attention (attention.hip) ---------------------------------------
int attn_num_splits(int rows, int k);
size_t attn_workspace_bytes(int B, int T, int H, int d_v, int k, dsa_dtype dtype);
dsa_status launch_attn_bf16(const void* q, const void* kv, const int32_t* idx, void* out,
                            float* lse, int B, int T, int N, int k, float sm_scale,
                            void* workspace, hipStream_t stream);
dsa_status launch_attn_f32(const float* q, const float* kv, const int32_t* idx, float* out,
                           float* lse, int B, int T, int N, int H, int d_qk, int d_v, int k,
                           float sm_scale, hipStream_t stream);

inline dsa_status launch_status() {
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // namespace dsa
