// LDS staging of K/V tiles shared by the MFMA kernels: buffer resources for the
// direct global->LDS loads and the XOR swizzles that keep the MFMA-side LDS reads
// free of bank conflicts.  Internal header.
#pragma once

#include "device_util.h"

namespace pa {

constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Buffer resource over [base, base + bytes): lanes whose offset falls outside read
// zeros (and, for the LDS-destination form, write zeros to LDS).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

// Raw buffer resource words over [base, base + bytes), for loads written in inline
// assembly.  User-space addresses are below 2^47, so the stride field stays zero.
__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kBufferFlags};
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from byte offset voffset of the buffer
// into LDS at lds_addr + 16 * lane; lanes whose offset lies outside the buffer write
// zeros and read nothing.  Written as inline assembly so the compiler does not track
// it (it would otherwise wait for these loads before unrelated LDS reads): callers
// wait with explicit vmcnt waits, and must have no compiler-visible vector memory
// loads of their own in flight while these are outstanding.
// The LDS address goes in through an M0 operand, so the compiler writes M0 itself and
// knows the asm reads it; the s_nop is the wait state between that write and the load.
__device__ __forceinline__ void lds_load16(u32x4 rsrc, uint32_t lds_addr, int voffset) {
  __asm__ __volatile__("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                       ::"{m0}"(lds_addr), "v"(voffset), "s"(rsrc) : "memory");
}

// LDS byte address of a __shared__ object, as M0 takes it.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt immediate for vmcnt(n) (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// XOR swizzles of the 16-byte chunks of an LDS row r holding D bf16 values.
//   K: chunk c of row r sits in slot c ^ (r mod chunks): the ds_read_b128 of 32
//      consecutive rows at one chunk hit distinct banks.
//   V: chunk c of row r sits in slot c ^ v_swizzle(r mod 4): the transposing
//      ds_read_b64_tr_b16 of 4 rows x 16 columns per 16 lanes hit distinct banks.
template <int D>
__device__ __forceinline__ int k_swizzle(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  const int x = r & 3;
  return D == 128 ? ((2 * x) ^ (8 * (x & 1))) : 2 * x;
}

}  // namespace pa
