// Arguments and launch set-up of the backward attention kernels. Everything
// that decides what one backward launch reads and writes, and in which order
// its workgroups run, lives in this header and in attn_bwd.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "attn_fwd_args.h"

namespace ra {

// Backward of one (query block, key block) pair, bf16 inputs. Element strides;
// rows of q/dout and k/v are contiguous (row stride D). The transposed copies
// qt/dot ([.., D, Cqp]) and kt ([.., D, Ckp]) and the per-row arrays
// lse2/ndelta ([.., Cqp]) are padded (zero columns / +inf, 0 rows).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const void* qt;      // Q^T
  const void* dot;     // dO^T
  const void* kt;      // K^T
  const float* lse2;   // lse * log2(e), +inf for rows without a key or padding
  const float* ndelta;  // minus <dout, out> per row, 0 for padding
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

// Head maps of a backward launch: head_order / kv_of from the (stable,
// KV-head-ordered) query head order and grp_off from the group sizes.
void fill_bwd_heads(BwdArgs& a, int32_t Hq, int32_t Hkv, const std::vector<uint8_t>& kv_of,
                    const std::vector<uint8_t>& order);

// The dk/dv kernel (a workgroup per 128 keys of one KV head) and the dq kernel
// (a workgroup per 256 queries of one query head); each sets its own work
// list (n_tiles, n_items, per_xcd) in its copy of the arguments.
hipError_t launch_bwd_dkdv(BwdArgs a, int D, hipStream_t s);
hipError_t launch_bwd_dq(BwdArgs a, int D, hipStream_t s);

}  // namespace ra
