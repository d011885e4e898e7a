// Helpers shared by the sparse-attention kernels (forward and backward):
// the latent-row swizzle of a gathered tile in LDS, bf16 MFMA, direct-to-LDS
// buffer loads and the XCD-aware workgroup order (gfx950 only).
#pragma once

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Row swizzle of the 16-byte chunks of a latent row: chunk c of tile row r
// sits in slot c ^ swz(r).  Eight consecutive rows read at one chunk hit
// eight different slots (the QK^T fragment reads), and the four rows x two
// chunks a 16-lane group touches in a transposed read are distinct as well.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& x) { return __builtin_bit_cast(bf16x8, x); }

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt left at "no wait")
#define DSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at p (raw buffer, 32-bit offsets; a load
// at an offset at or beyond `bytes` touches no memory and returns zeros).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* p, unsigned bytes) {
    const unsigned long long a = (unsigned long long)p;
    return i32x4{__builtin_amdgcn_readfirstlane((int)(unsigned)a),
                 __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes at buffer offset
// voff + soff land at lds_dst + 16*l.  Issued from inline assembly so that
// the compiler does not guard later LDS reads of other stages with waits on
// every load in flight; the ring waits for its own loads (vmcnt) before the
// barrier that publishes a stage.  No register receives data.
__device__ __forceinline__ void load_lds16(const i32x4& rsrc, unsigned lds_dst, unsigned voff,
                                           unsigned soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_dst), "v"(voff), "s"(rsrc), "s"(soff)
                 : "m0");
}

// 32-bit LDS address of a pointer into a __shared__ array
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(unsigned long long)(const __attribute__((address_space(3))) void*)p;
}

// Workgroups are dispatched round-robin over the chip's 8 XCDs (XCD = linear
// id % 8), each with its own L2.  Map linear ids so that every XCD works
// through a contiguous range of (query row, slot range) items: the slot
// ranges of one query row, which all read that row's Q, then run on one XCD.
// Ids past the last multiple of 8 keep their own number.
__device__ __forceinline__ unsigned xcd_contiguous(unsigned id, unsigned total) {
    const unsigned full = total & ~7u;
    if (id >= full) return id;
    return (id & 7u) * (full >> 3) + (id >> 3);
}

}  // namespace
}  // namespace dsa
