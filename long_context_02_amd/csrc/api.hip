// C ABI of libdsa: argument checks, workspace carving and kernel launches.
// Every entry point checks its arguments on the host before launching
// anything, never allocates, frees or synchronises, and reports launch
// failures as DSA_ERR_HIP.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "dsa_internal.h"

using namespace dsa;

// Scratch memory of dsa_forward_noalloc, for callers that cannot allocate a
// workspace: one fixed array per device, held from the library's load on
// that device until the process ends.  Every dsa_forward_noalloc call on a
// device uses (and overwrites) that device's array.
constexpr size_t kNoAllocScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxK = 2048;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dsa_status check_common(int B, int T, int N, int q_offset) {
    if (B < 1 || T < 1 || N < 1 || q_offset < 0) return DSA_ERR_INVALID_ARG;
    if ((long long)q_offset + T > N) return DSA_ERR_INVALID_ARG;
    if ((long long)B * T * (long long)N >= (1LL << 40)) return DSA_ERR_UNSUPPORTED;
    if (B > 65535) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

dsa_status check_indexer(const void* q_idx, const float* q_scale, const void* k_idx,
                         const float* k_scale, const float* w, const float* scores, int B, int T,
                         int N, int H_I, int d_I, int q_offset, dsa_dtype dt) {
    if (!q_idx || !k_idx || !w || !scores) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w) || !aligned16(scores))
        return DSA_ERR_INVALID_ARG;
    dsa_status st = check_common(B, T, N, q_offset);
    if (st != DSA_OK) return st;
    if (dt == DSA_FP8_E4M3FN) {
        if (!q_scale || !k_scale || !aligned16(q_scale) || !aligned16(k_scale))
            return DSA_ERR_INVALID_ARG;
        if (H_I != 8 || d_I != 128) return DSA_ERR_UNSUPPORTED;
        if (N >= (1 << 24)) return DSA_ERR_UNSUPPORTED;  // 32-bit byte offsets into keys and scores
        return DSA_OK;
    }
    if (dt == DSA_F32) {
        if (q_scale || k_scale) return DSA_ERR_INVALID_ARG;
        if (H_I < 1 || H_I > 16 || d_I < 1 || d_I > 256 || H_I * d_I > 4096) return DSA_ERR_UNSUPPORTED;
        if (T > 65535) return DSA_ERR_UNSUPPORTED;
        return DSA_OK;
    }
    return dt == DSA_BF16 ? DSA_ERR_UNSUPPORTED : DSA_ERR_INVALID_ARG;
}

dsa_status check_attn(const void* q, const void* kv, const int32_t* idx, const void* out,
                      const float* lse, int B, int T, int N, int H, int d_qk, int d_v, int k,
                      float sm_scale, dsa_dtype dt) {
    if (!q || !kv || !idx || !out) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(idx) || !aligned16(out) ||
        (lse && !aligned16(lse)))
        return DSA_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || N < 1 || k < 1) return DSA_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale)) return DSA_ERR_INVALID_ARG;
    if (k > kMaxK) return DSA_ERR_UNSUPPORTED;
    if (B > 65535 || T > 65535) return DSA_ERR_UNSUPPORTED;
    if ((long long)B * T > 0x7fffffffLL) return DSA_ERR_UNSUPPORTED;  // one workgroup id per row
    if ((long long)B * N * (long long)(d_qk > 0 ? d_qk : 1) >= (1LL << 42)) return DSA_ERR_UNSUPPORTED;
    if (dt == DSA_BF16) {
        if (H != 128 || d_qk != 576 || d_v != 512) return DSA_ERR_UNSUPPORTED;
        if ((long long)N * 1152 >= (1LL << 31)) return DSA_ERR_UNSUPPORTED;  // 32-bit row offsets
        return DSA_OK;
    }
    if (dt == DSA_F32) {
        if (H < 1 || H > 32 || d_qk < 1 || d_qk > 256 || d_v < 1 || d_v > d_qk) return DSA_ERR_UNSUPPORTED;
        return DSA_OK;
    }
    return dt == DSA_FP8_E4M3FN ? DSA_ERR_UNSUPPORTED : DSA_ERR_INVALID_ARG;
}

size_t attn_ws(int B, int T, int H, int d_v, int k) {
    const dsa_dtype dt = (H == 128 && d_v == 512) ? DSA_BF16 : DSA_F32;
    return attn_workspace_bytes(B, T, H, d_v, k, dt);
}

dsa_status run_indexer(const void* q_idx, const float* q_scale, const void* k_idx,
                       const float* k_scale, const float* w, float* scores, int B, int T, int N,
                       int H_I, int d_I, int q_offset, dsa_dtype dt, bool fill, hipStream_t s) {
    if (dt == DSA_FP8_E4M3FN)
        return launch_indexer_fp8(static_cast<const uint8_t*>(q_idx), q_scale,
                                  static_cast<const uint8_t*>(k_idx), k_scale, w, scores, B, T, N,
                                  q_offset, fill, s);
    return launch_indexer_f32(static_cast<const float*>(q_idx), static_cast<const float*>(k_idx),
                              w, scores, B, T, N, H_I, d_I, q_offset, fill, s);
}

// Workspace of the selection: the [B,T,N] fp32 scores, then the top-k
// workspace (per-row lists for batches of few rows).
size_t select_ws(int B, int T, int N, int k) {
    return align_up((size_t)B * T * N * sizeof(float)) + topk_workspace_bytes(B, T, N, k);
}

dsa_status run_select(const void* q_idx, const float* q_scale, const void* k_idx,
                      const float* k_scale, const float* w, int32_t* idx, int B, int T, int N,
                      int H_I, int d_I, int k, int q_offset, dsa_dtype dt, void* workspace,
                      hipStream_t s) {
    float* scores = static_cast<float*>(workspace);
    void* topk_ws = static_cast<char*>(workspace) + align_up((size_t)B * T * N * sizeof(float));
    if (dt == DSA_FP8_E4M3FN && indexer_filters(B, T)) {
        // decode-like batches: candidate lists from a sampled threshold
        // instead of the score matrix
        const auto* q8 = static_cast<const uint8_t*>(q_idx);
        const auto* k8 = static_cast<const uint8_t*>(k_idx);
        auto* sw = static_cast<uint32_t*>(topk_ws);
        dsa_status st = launch_indexer_sample_threshold(q8, q_scale, k8, k_scale, w, sw, B, T, N,
                                                        q_offset, k, s);
        if (st != DSA_OK) return st;
        st = launch_indexer_fp8_filtered(q8, q_scale, k8, k_scale, w, sw, B, T, N, q_offset, k, s);
        if (st != DSA_OK) return st;
        return launch_topk_from_candidates(q8, q_scale, k8, k_scale, w, scores, idx, B, T, N, k,
                                           q_offset, topk_ws, s);
    }
    dsa_status st = run_indexer(q_idx, q_scale, k_idx, k_scale, w, scores, B, T, N, H_I, d_I,
                                q_offset, dt, false, s);
    if (st != DSA_OK) return st;
    return launch_topk(scores, idx, B, T, N, k, q_offset, topk_ws, s);
}

dsa_status run_attn(const void* q, const void* kv, const int32_t* idx, void* out, float* lse,
                    int B, int T, int N, int H, int d_qk, int d_v, int k, float sm_scale,
                    dsa_dtype dt, void* ws, hipStream_t s) {
    if (dt == DSA_BF16) return launch_attn_bf16(q, kv, idx, out, lse, B, T, N, k, sm_scale, ws, s);
    return launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(kv), idx,
                           static_cast<float*>(out), lse, B, T, N, H, d_qk, d_v, k, sm_scale, s);
}

size_t forward_ws(int B, int T, int N, int H, int d_v, int k) {
    return align_up(select_ws(B, T, N, k)) + align_up((size_t)B * T * k * sizeof(int32_t)) +
           attn_ws(B, T, H, d_v, k);
}

// Argument checks of the fused path; *need receives its workspace bytes.
dsa_status check_forward(const void* q_idx, const float* q_idx_scale, const void* k_idx,
                         const float* k_idx_scale, const float* w, const void* q, const void* kv,
                         const void* out, const float* lse, const int32_t* idx_out, int B, int T,
                         int N, int H_I, int d_I, int H, int d_qk, int d_v, int k, int q_offset,
                         float sm_scale, dsa_dtype idx_dtype, dsa_dtype attn_dtype, size_t* need) {
    // the indexer's output goes to the workspace, so pass a stand-in for the check
    dsa_status st = check_indexer(q_idx, q_idx_scale, k_idx, k_idx_scale, w,
                                  reinterpret_cast<const float*>(16), B, T, N, H_I, d_I, q_offset,
                                  idx_dtype);
    if (st != DSA_OK) return st;
    st = check_attn(q, kv, reinterpret_cast<const int32_t*>(16), out, lse, B, T, N, H, d_qk, d_v, k,
                    sm_scale, attn_dtype);
    if (st != DSA_OK) return st;
    if (idx_out && !aligned16(idx_out)) return DSA_ERR_INVALID_ARG;
    *need = forward_ws(B, T, N, H, d_v, k);
    return DSA_OK;
}

// The fused path on a checked argument set and a workspace of at least
// forward_ws() bytes: selection, then attention.
dsa_status run_forward(const void* q_idx, const float* q_idx_scale, const void* k_idx,
                       const float* k_idx_scale, const float* w, const void* q, const void* kv,
                       void* out, float* lse, int32_t* idx_out, int B, int T, int N, int H_I,
                       int d_I, int H, int d_qk, int d_v, int k, int q_offset, float sm_scale,
                       dsa_dtype idx_dtype, dsa_dtype attn_dtype, void* workspace, hipStream_t s) {
    char* p = static_cast<char*>(workspace);
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(p + align_up(select_ws(B, T, N, k)));
    void* attn_w = p + align_up(select_ws(B, T, N, k)) + align_up((size_t)B * T * k * sizeof(int32_t));
    dsa_status st = run_select(q_idx, q_idx_scale, k_idx, k_idx_scale, w, idx, B, T, N, H_I, d_I, k,
                               q_offset, idx_dtype, workspace, s);
    if (st != DSA_OK) return st;
    return run_attn(q, kv, idx, out, lse, B, T, N, H, d_qk, d_v, k, sm_scale, attn_dtype, attn_w, s);
}

// ---- the fixed scratch array of dsa_forward_noalloc ----
// Device address of `scratch` on each device, looked up once per device
// (hipGetSymbolAddress with that device current).  In host code the name
// `scratch` is only a host-side handle of the symbol: kernels and copies get
// the address looked up here, never the name.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status noalloc_scratch(hipStream_t s, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
    if (s != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return DSA_ERR_HIP;
        if (sdev != dev) return DSA_ERR_INVALID_ARG;  // the stream must belong to the current device
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return DSA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_version(void) { return (1 << 16) | 3; }

const char* dsa_status_string(dsa_status s) {
    switch (s) {
        case DSA_OK: return "DSA_OK: success";
        case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape or dtype not supported";
        case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace too small";
        case DSA_ERR_BAD_INDEX: return "DSA_ERR_BAD_INDEX: index out of range";
        case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP launch failed";
    }
    return "unknown dsa_status";
}

size_t dsa_workspace_size(int op, int B, int T, int N, int H_I, int H, int d_v, int k) {
    if (B < 1 || T < 1 || N < 1 || k < 1 || k > kMaxK || H_I < 1 || H < 1 || d_v < 1)
        return (size_t)-1;
    switch (op) {
        case DSA_OP_TOPK: return topk_workspace_bytes(B, T, N, k);
        case DSA_OP_ATTN: return attn_ws(B, T, H, d_v, k);
        case DSA_OP_SELECT: return select_ws(B, T, N, k);
        case DSA_OP_ATTN_BWD: return attn_bwd_workspace_bytes(B, T, N, k);
        case DSA_OP_ATTN_MHA:
            if (H != 128 || d_v != 128) return (size_t)-1;
            return attn_mha_workspace_bytes(B, N);
        case DSA_OP_FORWARD: return forward_ws(B, T, N, H, d_v, k);
        default: return (size_t)-1;
    }
}

dsa_status dsa_indexer_scores(const void* q_idx, const float* q_idx_scale, const void* k_idx,
                              const float* k_idx_scale, const float* w, float* scores, int B,
                              int T, int N, int H_I, int d_I, int q_offset, dsa_dtype idx_dtype,
                              void* stream) {
    dsa_status st = check_indexer(q_idx, q_idx_scale, k_idx, k_idx_scale, w, scores, B, T, N, H_I,
                                  d_I, q_offset, idx_dtype);
    if (st != DSA_OK) return st;
    return run_indexer(q_idx, q_idx_scale, k_idx, k_idx_scale, w, scores, B, T, N, H_I, d_I,
                       q_offset, idx_dtype, true, static_cast<hipStream_t>(stream));
}

dsa_status dsa_topk_select(const float* scores, int32_t* idx, int B, int T, int N, int k,
                           int q_offset, void* workspace, size_t workspace_bytes, void* stream) {
    if (!scores || !idx || !aligned16(scores) || !aligned16(idx)) return DSA_ERR_INVALID_ARG;
    dsa_status st = check_common(B, T, N, q_offset);
    if (st != DSA_OK) return st;
    if (k < 1) return DSA_ERR_INVALID_ARG;
    if (k > kMaxK) return DSA_ERR_UNSUPPORTED;
    const size_t need = topk_workspace_bytes(B, T, N, k);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return DSA_ERR_WORKSPACE;
    return launch_topk(scores, idx, B, T, N, k, q_offset, workspace,
                       static_cast<hipStream_t>(stream));
}

dsa_status dsa_indexer_select(const void* q_idx, const float* q_idx_scale, const void* k_idx,
                              const float* k_idx_scale, const float* w, int32_t* idx, int B, int T,
                              int N, int H_I, int d_I, int k, int q_offset, dsa_dtype idx_dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
    // the scores go to the workspace, so pass a stand-in for the check
    dsa_status st = check_indexer(q_idx, q_idx_scale, k_idx, k_idx_scale, w,
                                  reinterpret_cast<const float*>(16), B, T, N, H_I, d_I, q_offset,
                                  idx_dtype);
    if (st != DSA_OK) return st;
    if (!idx || !aligned16(idx)) return DSA_ERR_INVALID_ARG;
    if (k < 1) return DSA_ERR_INVALID_ARG;
    if (k > kMaxK) return DSA_ERR_UNSUPPORTED;
    const size_t need = select_ws(B, T, N, k);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSA_ERR_WORKSPACE;
    return run_select(q_idx, q_idx_scale, k_idx, k_idx_scale, w, idx, B, T, N, H_I, d_I, k, q_offset,
                      idx_dtype, workspace, static_cast<hipStream_t>(stream));
}

dsa_status dsa_sparse_mla_attn(const void* q, const void* kv, const int32_t* idx, void* out,
                               float* lse, int B, int T, int N, int H, int d_qk, int d_v, int k,
                               float sm_scale, dsa_dtype attn_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
    dsa_status st = check_attn(q, kv, idx, out, lse, B, T, N, H, d_qk, d_v, k, sm_scale, attn_dtype);
    if (st != DSA_OK) return st;
    const size_t need = attn_workspace_bytes(B, T, H, d_v, k, attn_dtype);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return DSA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validation_enabled()) {
        st = validate_indices(idx, (size_t)B * T * k, N, s);
        if (st != DSA_OK) return st;
    }
    return run_attn(q, kv, idx, out, lse, B, T, N, H, d_qk, d_v, k, sm_scale, attn_dtype, workspace, s);
}

dsa_status dsa_sparse_mla_attn_bwd(const void* q, const void* kv, const int32_t* idx,
                                   const void* out, const float* lse, const void* dout, float* dq,
                                   float* dkv, int B, int T, int N, int H, int d_qk, int d_v, int k,
                                   float sm_scale, dsa_dtype attn_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    dsa_status st = check_attn(q, kv, idx, out, lse, B, T, N, H, d_qk, d_v, k, sm_scale, attn_dtype);
    if (st != DSA_OK) return st;
    if (!lse || !dout || !dq || !dkv) return DSA_ERR_INVALID_ARG;
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dkv)) return DSA_ERR_INVALID_ARG;
    if (attn_dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
    const size_t need = attn_bwd_workspace_bytes(B, T, N, k);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validation_enabled()) {
        st = validate_indices(idx, (size_t)B * T * k, N, s);
        if (st != DSA_OK) return st;
    }
    return launch_attn_bwd_bf16(q, kv, idx, out, lse, dout, dq, dkv, B, T, N, k, sm_scale, workspace, s);
}

dsa_status dsa_sparse_mla_attn_mha(const void* q, const void* kv, const void* w_uk,
                                   const void* w_uv, const int32_t* idx, void* out, float* lse,
                                   int B, int T, int N, int H, int d_c, int d_r, int d_n, int d_vh,
                                   int k, float sm_scale, dsa_dtype attn_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!q || !kv || !w_uk || !w_uv || !idx || !out) return DSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(idx) ||
        !aligned16(out) || (lse && !aligned16(lse)))
        return DSA_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || N < 1 || k < 1) return DSA_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale)) return DSA_ERR_INVALID_ARG;
    if (k > kMaxK) return DSA_ERR_UNSUPPORTED;
    if (attn_dtype != DSA_BF16) return attn_dtype == DSA_F32 || attn_dtype == DSA_FP8_E4M3FN
                                           ? DSA_ERR_UNSUPPORTED : DSA_ERR_INVALID_ARG;
    if (H != 128 || d_c != 512 || d_r != 64 || d_n != 128 || d_vh != 128) return DSA_ERR_UNSUPPORTED;
    if ((long long)B * T > 0x7fffffffLL || (long long)B * N >= (1LL << 31)) return DSA_ERR_UNSUPPORTED;
    const size_t need = attn_mha_workspace_bytes(B, N);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validation_enabled()) {
        const dsa_status st = validate_indices(idx, (size_t)B * T * k, N, s);
        if (st != DSA_OK) return st;
    }
    return launch_attn_mha_bf16(q, kv, w_uk, w_uv, idx, out, lse, B, T, N, k, sm_scale, workspace, s);
}

dsa_status dsa_forward(const void* q_idx, const float* q_idx_scale, const void* k_idx,
                       const float* k_idx_scale, const float* w, const void* q, const void* kv,
                       void* out, float* lse, int32_t* idx_out, int B, int T, int N, int H_I,
                       int d_I, int H, int d_qk, int d_v, int k, int q_offset, float sm_scale,
                       dsa_dtype idx_dtype, dsa_dtype attn_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
    size_t need = 0;
    dsa_status st = check_forward(q_idx, q_idx_scale, k_idx, k_idx_scale, w, q, kv, out, lse,
                                  idx_out, B, T, N, H_I, d_I, H, d_qk, d_v, k, q_offset, sm_scale,
                                  idx_dtype, attn_dtype, &need);
    if (st != DSA_OK) return st;
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSA_ERR_WORKSPACE;
    return run_forward(q_idx, q_idx_scale, k_idx, k_idx_scale, w, q, kv, out, lse, idx_out, B, T,
                       N, H_I, d_I, H, d_qk, d_v, k, q_offset, sm_scale, idx_dtype, attn_dtype,
                       workspace, static_cast<hipStream_t>(stream));
}

dsa_status dsa_forward_noalloc(const void* q_idx, const float* q_idx_scale, const void* k_idx,
                               const float* k_idx_scale, const float* w, const void* q,
                               const void* kv, void* out, float* lse, int32_t* idx_out, int B,
                               int T, int N, int H_I, int d_I, int H, int d_qk, int d_v, int k,
                               int q_offset, float sm_scale, dsa_dtype idx_dtype,
                               dsa_dtype attn_dtype, void* stream) {
    size_t need = 0;
    dsa_status st = check_forward(q_idx, q_idx_scale, k_idx, k_idx_scale, w, q, kv, out, lse,
                                  idx_out, B, T, N, H_I, d_I, H, d_qk, d_v, k, q_offset, sm_scale,
                                  idx_dtype, attn_dtype, &need);
    if (st != DSA_OK) return st;
    if (need > kNoAllocScratchBytes) return DSA_ERR_UNSUPPORTED;  // beyond the fixed scratch array
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    st = noalloc_scratch(s, &ws);
    if (st != DSA_OK) return st;
    return run_forward(q_idx, q_idx_scale, k_idx, k_idx_scale, w, q, kv, out, lse, idx_out, B, T,
                       N, H_I, d_I, H, d_qk, d_v, k, q_offset, sm_scale, idx_dtype, attn_dtype, ws,
                       s);
}

dsa_status dsa_cache_append(const float* k_new, const void* kv_new, void* k_cache,
                            float* k_cache_scale, void* kv_cache, const int32_t* pos, int B, int T,
                            int N, int d_I, int d_qk, dsa_dtype idx_dtype, dsa_dtype attn_dtype,
                            void* stream) {
    if (!k_new || !kv_new || !k_cache || !kv_cache || !pos) return DSA_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(kv_new) || !aligned16(k_cache) || !aligned16(kv_cache) ||
        !aligned16(pos) || (k_cache_scale && !aligned16(k_cache_scale)))
        return DSA_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || N < 1) return DSA_ERR_INVALID_ARG;
    if ((long long)B * N * 1152 >= (1LL << 46) || (long long)B * T >= (1LL << 31))
        return DSA_ERR_UNSUPPORTED;
    bool fp8;
    if (idx_dtype == DSA_FP8_E4M3FN) {
        if (!k_cache_scale) return DSA_ERR_INVALID_ARG;
        if (d_I != 128) return DSA_ERR_UNSUPPORTED;
        fp8 = true;
    } else if (idx_dtype == DSA_F32) {
        if (k_cache_scale) return DSA_ERR_INVALID_ARG;
        if (d_I < 1 || d_I > 256) return DSA_ERR_UNSUPPORTED;
        fp8 = false;
    } else {
        return idx_dtype == DSA_BF16 ? DSA_ERR_UNSUPPORTED : DSA_ERR_INVALID_ARG;
    }
    int row_bytes;
    if (attn_dtype == DSA_BF16) {
        if (d_qk != 576) return DSA_ERR_UNSUPPORTED;
        row_bytes = 576 * 2;
    } else if (attn_dtype == DSA_F32) {
        if (d_qk < 1 || d_qk > 256) return DSA_ERR_UNSUPPORTED;
        row_bytes = d_qk * 4;
    } else {
        return attn_dtype == DSA_FP8_E4M3FN ? DSA_ERR_UNSUPPORTED : DSA_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validation_enabled()) {
        const dsa_status st = validate_positions(pos, B, T, N, s);
        if (st != DSA_OK) return st;
    }
    return launch_cache_append(k_new, kv_new, k_cache, k_cache_scale, kv_cache, pos, B, T, N, d_I,
                               row_bytes, fp8, s);
}

dsa_status dsa_indexer_kl(const float* scores, const float* p, const int32_t* idx, float* loss,
                          float* grad, int B, int T, int N, int k, int q_offset, void* stream) {
    if (!scores || !p || !loss) return DSA_ERR_INVALID_ARG;
    if (!aligned16(scores) || !aligned16(p) || !aligned16(loss) || (grad && !aligned16(grad)) ||
        (idx && !aligned16(idx)))
        return DSA_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || N < 1) return DSA_ERR_INVALID_ARG;
    if ((long long)B * T >= (1LL << 31) || (long long)B * T * (long long)N >= (1LL << 40))
        return DSA_ERR_UNSUPPORTED;
    if (idx) {
        if (k < 1) return DSA_ERR_INVALID_ARG;
        if (k > kMaxK) return DSA_ERR_UNSUPPORTED;
    } else {
        if (q_offset < 0 || (long long)q_offset + T > N) return DSA_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (idx && validation_enabled()) {
        const dsa_status st = validate_indices(idx, (size_t)B * T * k, N, s);
        if (st != DSA_OK) return st;
    }
    return launch_indexer_kl(scores, p, idx, loss, grad, B, T, N, k, q_offset, s);
}

}  // extern "C"
