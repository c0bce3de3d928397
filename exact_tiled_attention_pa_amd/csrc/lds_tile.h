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
