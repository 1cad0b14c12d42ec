// Internal declarations shared by the gfx950 kernels and the host side of the
// ring-attention library. Not part of the public C ABI (include/ring_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ring_attn.h"

namespace ra {

// Attention workgroups: every wave64 owns 32 query rows. The bf16 kernel runs
// 8 waves (two groups of 4 that alternate MFMA and softmax phases), the fp32
// kernel 4 waves.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesBf16 = 8;
constexpr int kThreadsBf16 = 64 * kWavesBf16;
constexpr int kQTileF32 = 32 * kWaves;       // query rows per fp32 workgroup
constexpr int kQTileBf16 = 32 * kWavesBf16;  // query rows per bf16 workgroup
constexpr int kKTileBf16 = 64;       // keys per LDS tile, bf16 kernel
constexpr int kKTileF32 = 32;        // keys per LDS tile, fp32 kernel
constexpr int kVtAlign = 64;         // V^T rows are padded to a multiple of this
constexpr int kMaxHeads = 256;       // head maps travel in the kernel arguments
constexpr int kXcds = 8;             // MI355X: 8 XCDs, workgroups dealt round-robin

// Global positions of a block's rows: row t sits at
// start0 + t*stride (t < seg or nseg == 1) or start1 + (t - seg)*stride
// (nseg == 2). Positions increase with t and stay below 2^31.
struct PosDesc {
  int32_t nseg, seg, start0, start1, stride;
};

// Everything one attention launch needs. Strides are in elements; rows are
// contiguous (row stride D) except V^T, whose rows have length v_ld.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;          // bf16: V^T blocks [.., D, v_ld]; fp32: row-major V
  float* run_out;         // fp32 running output
  float* run_lse;         // fp32 running lse
  void* fin_out;          // non-null: final step, write out here in the input dtype
  float* fin_lse;         // final lse (used with fin_out)
  int64_t q_bs, q_hs;
  int64_t k_bs, k_hs;
  int64_t v_bs, v_hs, v_ld;
  int64_t ro_bs, ro_hs;
  int64_t rl_bs, rl_hs;
  int64_t fo_bs, fo_hs;
  int64_t fl_bs, fl_hs;
  int32_t B, Hq, Cq, Ck;
  PosDesc qp, kp;
  int32_t causal, accumulate;
  float scale;       // natural-units softmax scale
  float scale_log2;  // scale * log2(e)
  int32_t q_tile;    // query rows per workgroup (depends on the kernel)
  int32_t qt_lo;     // first query tile launched
  int32_t n_qt;      // query tiles launched per (b, head)
  int32_t n_items;   // B * Hq * n_qt
  int32_t per_xcd;   // ceil(n_items / kXcds)
  uint8_t head_order[kMaxHeads];  // query heads grouped by KV head
  uint8_t kv_of[kMaxHeads];       // KV head of each query head
};

hipError_t launch_attn(const AttnArgs& a, ra_dtype dt, int D, hipStream_t s);

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

}  // namespace ra
