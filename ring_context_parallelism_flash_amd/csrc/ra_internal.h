// Internal declarations shared by the gfx950 kernels and the host side of the
// ring-attention library. Not part of the public C ABI (include/ring_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_args.h"
#include "ring_attn.h"

namespace ra {

// Forward-kernel arguments, constants and PosDesc.


// Backward of one (query block, key block) pair, bf16 inputs. Element strides;
// rows of q/dout and k/v are contiguous (row stride D). The transposed copies
// qt/dot ([.., D, Cqp]) and kt ([.., D, Ckp]) and the per-row arrays
// lse2/delta ([.., Cqp]) are padded (zero columns / +inf, 0 rows).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const void* qt;      // Q^T
  const void* dot;     // dO^T
  const void* kt;      // K^T
  const float* lse2;   // lse * log2(e), +inf for rows without a key or padding
  const float* delta;  // <dout, out> per row, 0 for padding
  float* dq;           // fp32 accumulators (added to)
  float* dk;
  float* dv;
  int64_t q_bs, q_hs;    // q and dout
  int64_t k_bs, k_hs;    // k and v
  int64_t qt_bs, qt_hs;  // qt and dot (row length Cqp)
  int64_t kt_bs, kt_hs;  // kt (row length Ckp)
  int64_t l_bs, l_hs;    // lse2 and delta
  int64_t dq_bs, dq_hs;
  int64_t dk_bs, dk_hs;  // dk and dv
  int32_t B, Hq, Hkv, Cq, Ck, Cqp, Ckp;
  PosDesc qp, kp;
  int32_t causal;
  float scale;       // natural-units softmax scale
  float scale_log2;  // scale * log2(e)
  int32_t n_tiles;   // key tiles (dk/dv kernel) or query tiles (dq kernel) per head
  int32_t n_items;
  int32_t per_xcd;
  uint8_t head_order[kMaxHeads];   // query heads grouped by KV head
  uint8_t kv_of[kMaxHeads];
  uint16_t grp_off[kMaxHeads + 1];  // head_order[grp_off[g] .. grp_off[g+1]) read KV head g
};

constexpr int kBwdRowPad = 128;  // padding of the row counts Cqp, Ckp

hipError_t launch_bwd_dkdv(const BwdArgs& a, int D, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int D, hipStream_t s);

// delta[row] = <dout, out> and lse2[row] = lse * log2(e) (+inf for -inf) for
// rows (bh, blk, i), i < C, of [BH][nblk*C][D] bf16 arrays (bh stride o_bh
// elements; lse bh stride l_bh); written to [BH][nblk][Cp] with padding rows
// i >= C set to delta 0, lse2 +inf.
hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* lse2p,
                           float* deltap, int64_t BH, int64_t nblk, int64_t C, int64_t Cp, int D,
                           int64_t o_bh, int64_t l_bh, hipStream_t s);

// dst[i] = bf16(src[i]) (round to nearest even), n a multiple of 4.
hipError_t launch_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t s);

// v: [BH][nblk*C][D] bf16 with per-bh stride v_bh (elements) -> vt:
// [BH][nblk][D][Cpad] bf16, zero for columns C..Cpad-1.
hipError_t launch_vt_transpose(const void* v, void* vt, int64_t BH, int64_t nblk, int64_t C,
                               int64_t Cpad, int D, int64_t v_bh, hipStream_t s);

hipError_t launch_lse_merge(float* out, float* lse, const float* out_b, const float* lse_b,
                            int64_t rows, int D, hipStream_t s);

hipError_t launch_zigzag_permute(const void* src, void* dst, int64_t outer, int64_t S,
                                 int64_t row_bytes, int N, int inverse, hipStream_t s);

hipError_t launch_striped_permute(const void* src, void* dst, int64_t outer, int64_t S,
                                  int64_t row_bytes, int N, int inverse, hipStream_t s);
hipError_t launch_ulysses_a2a(const void* src, void* dst, int32_t B, int64_t S, int32_t H,
                              int64_t row_bytes, int32_t P, int inverse, hipStream_t s);

}  // namespace ra
