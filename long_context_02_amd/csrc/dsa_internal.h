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

// ---- top-k selection key and the per-row workspace of few-row selection ----
// Order-preserving map float -> uint32 (larger float -> larger key); -0 and
// +0 map to one key, NaN to the lowest.
__device__ __forceinline__ uint32_t fkey(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0u) return 0x80000000u;
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Batches of at most seg::kMaxRows rows select with several workgroups per
// row.  Row r owns seg::kRowWords 32-bit words of the top-k workspace: a
// histogram of the top 12 key bits, four counters (sure picks, candidates,
// candidate overflow flag, candidate threshold key), the list of sure picks
// and the candidate list (keys, then token indices).
namespace seg {
constexpr int kMaxRows = 255;
constexpr int kBins = 4096;
constexpr int kMaxK = 2048;
constexpr int kCap = 12288;  // candidates per row
constexpr int kHist = 0, kCtr = kBins, kTheta = kCtr + 3, kDef = kBins + 4, kCKey = kDef + kMaxK,
              kCIdx = kCKey + kCap;
constexpr int kRowWords = (kCIdx + kCap + 63) / 64 * 64;
}  // namespace seg
inline bool topk_segmented(long long rows) { return rows <= seg::kMaxRows; }

// ---- indexer (indexer.hip) ------------------------------------------------
// fill_masked: write -inf over the non-causal part of every row (the public
// entry point promises that); the fused path skips those stores.
dsa_status launch_indexer_fp8(const uint8_t* q, const float* qs, const uint8_t* k,
                              const float* ks, const float* w, float* scores,
                              int B, int T, int N, int q_offset, bool fill_masked,
                              hipStream_t stream);
// Decode selection without a score matrix (batches with T < 16 and at most
// seg::kMaxRows rows): a per-row candidate threshold from a sample of keys,
// then the stream indexer appending only keys at or above it to the rows'
// candidate lists in seg_ws (the top-k workspace); scores is not written.
bool indexer_filters(int B, int T);
dsa_status launch_indexer_sample_threshold(const uint8_t* q, const float* qs, const uint8_t* k,
                                           const float* ks, const float* w, uint32_t* seg_ws,
                                           int B, int T, int N, int q_offset, int top_k,
                                           hipStream_t stream);
dsa_status launch_indexer_fp8_filtered(const uint8_t* q, const float* qs, const uint8_t* k,
                                       const float* ks, const float* w, uint32_t* seg_ws,
                                       int B, int T, int N, int q_offset, int top_k,
                                       hipStream_t stream);
dsa_status launch_indexer_f32(const float* q, const float* k, const float* w, float* scores,
                              int B, int T, int N, int H_I, int d_I, int q_offset,
                              bool fill_masked, hipStream_t stream);

// ---- top-k (topk.hip) -----------------------------------------------------
size_t topk_workspace_bytes(int B, int T, int N, int k);
dsa_status launch_topk(const float* scores, int32_t* idx, int B, int T, int N, int k,
                       int q_offset, void* workspace, hipStream_t stream);
// Selection from the candidate lists the filtered indexer built in the top-k
// workspace; a row whose list cannot be trusted (fewer than k candidates or
// an overflow) is rescored into scores (the caller's [B,T,N] buffer) and
// selected from there.
dsa_status launch_topk_from_candidates(const uint8_t* q, const float* qs, const uint8_t* k,
                                       const float* ks, const float* w, float* scores,
                                       int32_t* idx, int B, int T, int N, int top_k, int q_offset,
                                       void* workspace, hipStream_t stream);

// ---- sparse attention (attention.hip) ---------------------------------------
int attn_num_splits(int rows, int k);
size_t attn_workspace_bytes(int B, int T, int H, int d_v, int k, dsa_dtype dtype);
dsa_status launch_attn_bf16(const void* q, const void* kv, const int32_t* idx, void* out,
                            float* lse, int B, int T, int N, int k, float sm_scale,
                            void* workspace, hipStream_t stream);
dsa_status launch_attn_f32(const float* q, const float* kv, const int32_t* idx, float* out,
                           float* lse, int B, int T, int N, int H, int d_qk, int d_v, int k,
                           float sm_scale, hipStream_t stream);

// ---- sparse attention in MHA mode (attention_mha.hip) ------------------------
// bf16 only: H = 128, latent 512 + rope 64, per-head key 128 + 64, value 128.
// The workspace holds the up-projected per-head keys [B,N,H,192] and values
// [B,N,H,128] (bf16) of every latent row.
size_t attn_mha_workspace_bytes(int B, int N);
dsa_status launch_attn_mha_bf16(const void* q, const void* kv, const void* w_uk, const void* w_uv,
                                const int32_t* idx, void* out, float* lse, int B, int T, int N,
                                int k, float sm_scale, void* workspace, hipStream_t stream);

// ---- sparse attention backward (attention_bwd.hip) --------------------------
// bf16 only (H = 128, d_qk = 576, d_v = 512).  dq [B,T,H,576] and dkv
// [B,N,576] are fp32 and fully overwritten; the workspace holds one block of
// rows' P and dS tiles, latent-gradient contribution rows and the per-token
// lists, plus per-token counts and offsets.
size_t attn_bwd_workspace_bytes(int B, int T, int N, int k);
dsa_status launch_attn_bwd_bf16(const void* q, const void* kv, const int32_t* idx, const void* out,
                                const float* lse, const void* dout, float* dq, float* dkv, int B,
                                int T, int N, int k, float sm_scale, void* workspace,
                                hipStream_t stream);

// ---- cache append (cache.hip) ---------------------------------------------
// fp8: quantise the key rows (d_i = 128) into codes + scales; otherwise copy
// f32 key rows.  Latent rows are copied as kv_row_bytes bytes.
dsa_status launch_cache_append(const float* k_new, const void* kv_new, void* k_cache, float* k_scale,
                               void* kv_cache, const int32_t* pos, int B, int T, int N, int d_i,
                               int kv_row_bytes, bool fp8, hipStream_t stream);

// ---- indexer KL objective (kl.hip) -----------------------------------------
// idx == nullptr: dense rows (p, grad [B,T,N], causal range from q_offset);
// otherwise the k selected slots of each row (p, grad [B,T,k]).  grad may be
// nullptr.
dsa_status launch_indexer_kl(const float* scores, const float* p, const int32_t* idx, float* loss,
                             float* grad, int B, int T, int N, int k, int q_offset, hipStream_t stream);

// ---- debug validation of caller indices (validate.hip) -----------------------
// validation_enabled(): the environment holds DSA_VALIDATE=1 (read per call).
// The validators count bad entries on stream s, wait for it and return
// DSA_ERR_BAD_INDEX if there are any.
bool validation_enabled();
dsa_status validate_indices(const int32_t* idx, size_t n, int N, hipStream_t s);
dsa_status validate_positions(const int32_t* pos, int B, int T, int N, hipStream_t s);

// ---- per-kernel timing (profile.hip) -----------------------------------------
// While dsa_profile_start's window is open, a Scope records a HIP event on
// its stream when constructed and another when destroyed; DSA_TIMED wraps one
// kernel launch in such a scope.  Names are static strings.
namespace prof {
bool enabled();
class Scope {
  public:
    Scope(const char* name, hipStream_t s);
    ~Scope();
  private:
    int slot_;
    hipStream_t stream_;
};
dsa_status open_window(int max_launches);
int close_window(dsa_kernel_time* out, int max_out, int* dropped);
}  // namespace prof
#define DSA_TIMED(name, stream, ...)                       \
    do {                                                  \
        ::dsa::prof::Scope dsa_timed_scope_(name, stream); \
        __VA_ARGS__;                                      \
    } while (0)

inline dsa_status launch_status() {
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // namespace dsa
