// Helpers shared by the kernels that stream a weight through a ring of LDS
// stages filled by direct-to-LDS loads (global_load_lds) on gfx950: the
// vocabulary GEMMs, the decode-step head and the expert GEMMs.
#pragma once

#include <cstdint>

namespace dg {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// vmcnt(n): wait until at most n vector-memory operations of this wave are
// outstanding; lgkm and exp counters are left alone.
#define DG_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | ((((n) >> 4) & 3) << 14))

// Barrier that only waits for this wave's LDS traffic: the direct-to-LDS
// loads of later stages stay in flight across it.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
}

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row: chunk c of
// row r sits in slot c ^ swz(r).  A fragment read (ds_read_b128; lane l
// reads row l % 16, chunk l / 16) then runs at the rate of a linear 1 KiB
// read: measured on gfx950, 4.5 LDS cycles per instruction and CU against
// 8.4 unswizzled, and 8.4 as well with (r >> 3) also folded in.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

}  // namespace dg
