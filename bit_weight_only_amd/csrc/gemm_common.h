// Building blocks of the MFMA dequant-GEMM kernels: asynchronous global -> LDS
// copies, explicit vector-memory waits, the 4x4 lane transpose that hands each
// lane its word column of four 16-byte code vectors, and the device-coherent
// loads and stores of split-K partial tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbq {

// Transpose a 4x4 matrix held as element e of lanes in 16-lane row r: after
// the call, element e of lane (j, row r) is the old element r of lane (j, row e).
__device__ __forceinline__ void transpose4(uint32_t &e0, uint32_t &e1, uint32_t &e2, uint32_t &e3) {
  const auto a = __builtin_amdgcn_permlane32_swap(e0, e2, false, false);
  e0 = a[0];
  e2 = a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(e1, e3, false, false);
  e1 = b[0];
  e3 = b[1];
  const auto c = __builtin_amdgcn_permlane16_swap(e0, e1, false, false);
  e0 = c[0];
  e1 = c[1];
  const auto d = __builtin_amdgcn_permlane16_swap(e2, e3, false, false);
  e2 = d[0];
  e3 = d[1];
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// Asynchronous copies global -> LDS (global_load_lds): lane l of the wave
// sends 16 (4) bytes from its own address src to dst_base + 16 l (4 l);
// dst_base must be the same for the whole wave. Counted by the vector-memory
// counter.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *dst_base) {
  __builtin_amdgcn_global_load_lds((global_void_t *)src, (lds_void_t *)dst_base, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const void *src, void *dst_base) {
  __builtin_amdgcn_global_load_lds((global_void_t *)src, (lds_void_t *)dst_base, 4, 0, 0);
}

// s_waitcnt: at most N vector-memory operations of this wave outstanding, and
// every LDS operation done (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS accesses only. __syncthreads() also waits
// for every global load the wave has in flight (its fence covers global memory),
// which drains a prefetch ring at the barrier; here only this wave's LDS
// operations complete first (the fences name the local address space), and the
// ring's loads stay in flight across it. For data the waves exchange through
// LDS written with ds_* stores (copies into LDS by global_load_lds are counted
// by vmcnt and need wait_vm_lds).
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Partial tiles cross workgroups (and L2 slices): agent-scope relaxed atomics
// read and write them at the device-coherent level, so no cache flush or
// invalidate is needed; a wait for the stores' completion orders them before
// the arrival counter.
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace lbq
