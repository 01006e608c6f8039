// Device helpers shared by the GEMM kernels: LDS DMA copies with explicit waits, the
// workgroup barrier after a wave's LDS reads, and the XCD-aware tile order.
#pragma once
#include "common.h"

namespace svdq {

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));


// 16 B per lane from sbase + voff to LDS byte address lds + 16 * lane (the LDS
// address travels in M0; one wait state separates its write from the load).  Written as
// asm so that the compiler neither reorders LDS accesses around it (memory clobber)
// nor inserts its own conservative vmcnt waits; the waits are the explicit
// wait_vm below.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier once this wave's LDS reads are complete.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const void lds_void;
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)p);
}

// Partial tile of tail tile t, piece p in the split area.
__device__ __forceinline__ float* part_tile(float* part, int t, int p, int ks, int tile_floats) {
  return part + (size_t)(t * ks + p) * tile_floats;
}

// Tile (tm, tn) of tile id t: XCD-aware when the grid allows (t % 8 is the XCD that
// workgroup t runs on; XCD x takes a (tiles_m / 4) x (tiles_n / 2) sub-grid), else
// row-major.

__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  if (tiles_m % 4 == 0 && tiles_n % 2 == 0) {
    const int x = t & 7, loc = t >> 3;
    const int sm = tiles_m >> 2, sn = tiles_n >> 1;
    tm = (x >> 1) * sm + loc / sn;
    tn = (x & 1) * sn + loc % sn;
  } else {
    tn = t % tiles_n;
    tm = t / tiles_n;
  }
}


// Waits until at most N of this wave's vector memory operations (LDS DMA copies
// included) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace svdq
