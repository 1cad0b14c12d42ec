// Device helpers shared by the attention kernels (forward and backward):
// vector types, position descriptors and the causal rule, the score-row
// permutation that lets MFMA results feed the next MFMA directly, and the
// LDS load / read primitives.
#pragma once

#include <math.h>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int pos_of(const PosDesc& p, int t) {
  const bool second = (p.nseg == 2) & (t >= p.seg);
  return second ? p.start1 + (t - p.seg) * p.stride : p.start0 + t * p.stride;
}

// Score with the causal / ragged mask applied, as a select. The mask is
// evaluated without short-circuit branches on purpose: a divergent
// short-circuit condition guarding a store into one element of an MFMA
// accumulator vector was compiled into code that dropped the store.
__device__ __forceinline__ float masked(float s, int key, int Ck, int causal, const PosDesc& kp,
                                        int qpos) {
  const bool ok = (key < Ck) & ((causal == 0) | (pos_of(kp, min(key, Ck - 1)) <= qpos));
  return ok ? s : -INFINITY;
}


// Number of keys whose position is <= P. Positions increase with the row
// index, so these keys are a prefix of the block.
__device__ __forceinline__ int allowed_prefix(const PosDesc& p, int P) {
  // rows i < seg of a segment starting at s with s + i*stride <= P
  const int n0 = P < p.start0 ? 0 : min((P - p.start0) / p.stride + 1, p.seg);
  const int n1 = (p.nseg == 2 && P >= p.start1) ? min((P - p.start1) / p.stride + 1, p.seg) : 0;
  return n0 + n1;
}

// Row of the K tile that feeds MFMA row m of a 32-key S^T tile (bf16 kernel).
// MFMA output row m = 4*h + (j%4) + 8*(j/4) + 16*w (h = lane half, j = slot)
// is sent to key 16*w + 8*h + j, so lane half h ends up holding keys
// {8h..8h+7, 16+8h..16+8h+7}: one 16-byte V^T read per PV step.
__device__ __forceinline__ int kperm(int m) {
  const int w = m >> 4, r = m & 15;
  return 16 * w + 8 * ((r >> 2) & 1) + (r & 3) + 4 * (r >> 3);
}

// One wave-wide direct global->LDS load: lane i's 16 bytes land at
// lds_base + 16*i (lds_base must be the same for the whole wave).
__device__ __forceinline__ void load_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Barrier that also publishes this wave's direct global->LDS loads. The
// compiler does not count those loads as LDS writes a barrier must wait for
// (it emitted a bare s_barrier inside the key loop), so the vector-memory
// counter is drained explicitly first.
__device__ __forceinline__ void lds_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Workgroup barrier without the memory fence of __syncthreads(). That fence
// makes the compiler wait for every outstanding vector-memory operation --
// including direct global->LDS tile loads meant to stay in flight across the
// barrier. Callers wait explicitly for what the barrier publishes: their own
// tile loads (vmcnt) and their LDS reads (lgkmcnt, the operand rings wait for
// every read they issue). The "memory" clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

// This lane's index in the wave, computed by volatile asm: an expression of
// it cannot be hoisted out of a loop (a hoisted per-lane value stays live in
// a register through the loop).
__device__ __forceinline__ int lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// 32-bit LDS address of a pointer into this workgroup's LDS.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// Explicitly ordered LDS operand stream. The compiler keeps at most one or
// two operand reads in flight ahead of the MFMAs (it recycles one register
// set and drains the LDS counter); issuing the reads here, into a ring of
// registers, with an explicit wait before each use keeps several in flight.
// The wait names the register it guards, so its consumer cannot be moved
// above it.
template <int OFF>
__device__ __forceinline__ bf16x8 ds_read16(unsigned addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait(bf16x8& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N) : "memory");
}

}  // namespace
}  // namespace ra
