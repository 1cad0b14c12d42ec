// Internal declarations shared by the gfx950 kernels and the host side of the
// ring-attention library. Not part of the public C ABI (include/ring_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bwd_args.h"
#include "attn_fwd_args.h"
#include "ring_attn.h"

namespace ra {

// Forward-kernel arguments, constants and PosDesc.


// Backward-kernel arguments: attn_bwd_args.h.

// delta[row] = <dout, out> and lse2[row] = lse * log2(e) (+inf for -inf) for
// rows (bh, blk, i), i < C, of [BH][nblk*C][D] bf16 arrays (bh stride o_bh
// elements; lse bh stride l_bh); written to [BH][nblk][Cp] with padding rows
// i >= C set to 0, lse2 +inf. ndeltap receives minus delta.
hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* lse2p,
                           float* ndeltap, int64_t BH, int64_t nblk, int64_t C, int64_t Cp, int D,
                           int64_t o_bh, int64_t l_bh, hipStream_t s);

// dst[i] = bf16(src[i]) (round to nearest even), n a multiple of 4.
hipError_t launch_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t s);

// v: [BH][nblk*C][D] bf16 with per-bh stride v_bh (elements) -> vt:
// [BH][nblk][D][Cpad] bf16, zero for columns C..Cpad-1.
hipError_t launch_vt_transpose(const void* v, void* vt, int64_t BH, int64_t nblk, int64_t C,
                               int64_t Cpad, int D, int64_t v_bh, hipStream_t s);

// Zero `bytes` bytes at p (16-byte aligned, bytes a multiple of 16) with a
// kernel, so a captured stream records a kernel node rather than a memset.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);

hipError_t launch_lse_merge(float* out, float* lse, const float* out_b, const float* lse_b,
                            int64_t rows, int D, hipStream_t s);

hipError_t launch_zigzag_permute(const void* src, void* dst, int64_t outer, int64_t S,
                                 int64_t row_bytes, int N, int inverse, hipStream_t s);

hipError_t launch_striped_permute(const void* src, void* dst, int64_t outer, int64_t S,
                                  int64_t row_bytes, int N, int inverse, hipStream_t s);
// Ulysses all-to-all: [P][B][S/P][H] rows <-> [P][B][H/P][S] rows; the
// head-sharded side's head planes start every hs_stride rows (<= 0: S) at
// row offset hs_off.
hipError_t launch_ulysses_a2a(const void* src, void* dst, int32_t B, int64_t S, int32_t H,
                              int64_t row_bytes, int32_t P, int inverse, hipStream_t s,
                              int64_t hs_stride = 0, int64_t hs_off = 0);

// Matrix-core probe: one workgroup of kProbeThreads per compute unit (the
// dynamic LDS request leaves room for one); writes kProbeWords int64 per wave
// (shader-clock counter at start and end, 100 MHz reference counter at start
// and end, a liveness word) to out.
constexpr int kProbeThreads = 512;
constexpr int kProbeWords = 5;
constexpr size_t kProbeLdsBytes = 96 * 1024;
hipError_t launch_mfma_probe(int32_t workgroups, int32_t iters, int64_t* out, hipStream_t s);

// Static device scratch of ra_block_attn_fwd_noalloc (64 MiB per device):
// *ptr receives the current device's address of the array, looked up once
// per device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace ra
