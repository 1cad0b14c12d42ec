// Arguments and launch set-up of the forward attention kernels. Everything
// that decides what one forward launch reads and writes, and in which order
// its workgroups run, lives in this header and in attn_fwd.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

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
  alignas(4) uint8_t head_order[kMaxHeads];  // query heads grouped by KV head
  alignas(4) uint8_t kv_of[kMaxHeads];       // KV head of each query head
};

hipError_t launch_attn(const AttnArgs& a, ra_dtype dt, int D, hipStream_t s);

// Work list of a forward launch: fills B, Hq, q_tile, qt_lo, n_qt, n_items,
// per_xcd and the head maps (query heads ordered by KV head in `order`). With
// causal, accumulate and no final output, leading query tiles that see no key
// are skipped. Needs a.qp, a.kp, a.Ck, a.causal, a.accumulate, a.fin_out set.
void fill_attn_work(AttnArgs& a, ra_dtype dt, int32_t B, int32_t Hq, int64_t Cq,
                    const std::vector<uint8_t>& kv_of, const std::vector<uint8_t>& order);

}  // namespace ra
