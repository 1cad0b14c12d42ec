// Blockwise attention of one query block against one KV block, merged into a
// running (out, lse) state -- the per-step kernel of ring attention.
//
// Method: "Context Parallelism" (aiwiki), ring_attention listing (flash_block
// with a source-dependent mask) and "Ring attention" (exact, blockwise);
// "Sequence Parallelism in Large Language Models ..." (llms.blog),
// "Algorithmic Mechanics" (online-softmax running max / sum / rescaled output)
// and "Causal Masking and Load Balancing" (j <= i on global positions).
//
// gfx950 design
//  * D = 128 bf16 blocks of whole 64-key tiles run attn_fwd_bf16_w64: one
//    wave per SIMD owns 64 query rows (two 32-row blocks), so every K or V^T
//    operand read from LDS feeds two MFMAs; its key loop is one generated
//    inline-asm statement (attn_fwd_w64_phases.h, gen_fwd_w64.py) that
//    interleaves each block's softmax with the other MFMA phase.
//  * Other bf16 blocks (D = 64, ragged blocks) run attn_fwd_bf16: each wave64
//    owns 32 query rows, 8 waves (256 rows) per workgroup in two groups that
//    alternate matrix and softmax phases; the fp32 kernel runs 4 waves (128
//    rows).
//  * Scores are computed transposed, S^T = K * Q^T, with
//    v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query, so the
//    row max and row sum of the online softmax are in-lane reductions plus a
//    single exchange with the lane 32 away. Q stays in registers.
//  * The output is accumulated transposed too, O^T += V^T * P^T: the fp32
//    score registers, rounded to bf16, are directly the B operand (no
//    shuffles), and the per-query rescale factor is in-lane.
//  * K is staged in LDS as [key][d]; V is staged as V^T [d][key] (the host
//    transposes V once per call) so both MFMA operands are 16-byte LDS reads.
//    The rows of each 32-key S^T tile are permuted so that the keys a lane
//    holds after the first MFMA are exactly the 8 consecutive keys its V^T
//    operand needs in the second.
//  * Key tiles are classified from global positions: tiles past the causal
//    frontier are never visited, fully visible tiles skip the mask, and only
//    the diagonal / ragged tiles evaluate a per-element mask.
//  * Workgroup ids are remapped so each XCD (ids dealt round-robin over 8
//    XCDs) runs a contiguous range of (head, query tile) items: query heads
//    that share a KV head, and neighbouring query tiles, then read the same
//    K/V tiles through that XCD's L2.
//  * The fp32 kernel (v_mfma_f32_32x32x2_f32) keeps the same structure with
//    one element per lane per operand, so V needs no transpose there.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "attn_fwd_w64_phases.h"

namespace ra {
namespace {

struct WorkItem {
  int b, h, g, q0;
};

__device__ __forceinline__ bool decode_item(const AttnArgs& a, WorkItem& it) {
  const int w = blockIdx.x;
  const int L = (w % kXcds) * a.per_xcd + (w / kXcds);
  if (L >= a.n_items) return false;
  const int qt_rel = L % a.n_qt;
  const int rest = L / a.n_qt;
  const int hidx = rest % a.Hq;
  it.b = rest / a.Hq;
  // The head tables are read as 32-bit words of the kernel arguments, and
  // the results marked uniform, so the pointers derived from them stay in
  // scalar registers.
  const uint32_t* ho = reinterpret_cast<const uint32_t*>(a.head_order);
  const uint32_t* ko = reinterpret_cast<const uint32_t*>(a.kv_of);
  it.h = __builtin_amdgcn_readfirstlane((int)((ho[hidx >> 2] >> (8 * (hidx & 3))) & 255u));
  it.g = __builtin_amdgcn_readfirstlane((int)((ko[it.h >> 2] >> (8 * (it.h & 3))) & 255u));
  // heaviest (latest-position) query tiles first
  it.q0 = (a.qt_lo + (a.n_qt - 1 - qt_rel)) * a.q_tile;
  return true;
}

// Online-softmax update for one key tile, on the scores of one lane. S holds
// NSC score vectors of 16; masked entries are -inf. Returns the scale that was
// applied to the running output (alpha) and turns S into probabilities.
template <int NSC>
__device__ __forceinline__ float softmax_tile(floatx16 (&S)[NSC], float& m_run, float& l_part,
                                              float scale_log2) {
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NSC; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[t][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
  const float moff = m_use * scale_log2;
  float rs = 0.f;
#pragma unroll
  for (int t = 0; t < NSC; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(S[t][i], scale_log2, -moff));
      S[t][i] = p;
      rs += p;
    }
  l_part = l_part * alpha + rs;
  m_run = m_new;
  return alpha;
}

// Merge the block result into the running state (or write it) for the lane's
// query row. O holds the unnormalised O^T accumulators: lane (n, hh) holds
// d = 32*T + 4*hh + (i%4) + 8*(i/4) of query n.
template <int DT, bool BF16>
__device__ __forceinline__ void epilogue(const AttnArgs& a, const WorkItem& it, int qi, int hh,
                                         floatx16 (&O)[DT], float m_run, float l_part) {
  constexpr int D = DT * 32;
  const float l = l_part + __shfl_xor(l_part, 32);
  if (qi >= a.Cq) return;
  const bool fin = a.fin_out != nullptr;
  const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
  const float lse_blk = (l > 0.f) ? fmaf(m_use, a.scale, logf(l)) : -INFINITY;
  if (a.accumulate && lse_blk == -INFINITY && !fin) return;  // nothing to fold in

  float* ro = a.run_out + it.b * a.ro_bs + it.h * a.ro_hs + (int64_t)qi * D;
  float* rl = a.run_lse + it.b * a.rl_bs + it.h * a.rl_hs + qi;
  const float lse_old = a.accumulate ? *rl : -INFINITY;
  const float mx = fmaxf(lse_old, lse_blk);
  float lse_new, ca, cb;
  if (mx == -INFINITY) {
    lse_new = -INFINITY;
    ca = 0.f;
    cb = 0.f;
  } else {
    const float mn = fminf(lse_old, lse_blk);
    lse_new = mx + log1pf(expf(mn - mx));
    ca = (lse_old == -INFINITY) ? 0.f : expf(lse_old - lse_new);
    cb = (lse_blk == -INFINITY) ? 0.f : expf(lse_blk - lse_new) / l;
  }

#pragma unroll
  for (int T = 0; T < DT; ++T)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * T + 8 * g4 + 4 * hh;
      float4 r;
      r.x = O[T][4 * g4 + 0] * cb;
      r.y = O[T][4 * g4 + 1] * cb;
      r.z = O[T][4 * g4 + 2] * cb;
      r.w = O[T][4 * g4 + 3] * cb;
      if (ca != 0.f) {
        const float4 old = *reinterpret_cast<const float4*>(ro + d0);
        r.x = fmaf(old.x, ca, r.x);
        r.y = fmaf(old.y, ca, r.y);
        r.z = fmaf(old.z, ca, r.z);
        r.w = fmaf(old.w, ca, r.w);
      }
      if (fin) {
        if constexpr (BF16) {
          __bf16* fo = reinterpret_cast<__bf16*>(a.fin_out) + it.b * a.fo_bs + it.h * a.fo_hs +
                       (int64_t)qi * D + d0;
          bf16x4 pk;
          pk[0] = (__bf16)r.x;
          pk[1] = (__bf16)r.y;
          pk[2] = (__bf16)r.z;
          pk[3] = (__bf16)r.w;
          *reinterpret_cast<bf16x4*>(fo) = pk;
        } else {
          float* fo = reinterpret_cast<float*>(a.fin_out) + it.b * a.fo_bs + it.h * a.fo_hs +
                      (int64_t)qi * D + d0;
          *reinterpret_cast<float4*>(fo) = r;
        }
      } else {
        *reinterpret_cast<float4*>(ro + d0) = r;
      }
    }
  if (hh == 0) {
    if (fin)
      a.fin_lse[it.b * a.fl_bs + it.h * a.fl_hs + qi] = lse_new;
    else
      *rl = lse_new;
  }
}

// The same merge for the two 32-row blocks of a one-wave-per-SIMD wave (bf16
// inputs, D = 128; ACC: fold into the running state, FIN: write the final
// output), through the wave's own LDS staging area so that the running state
// is read and written in whole rows (each 16-byte access of the MFMA layout
// would otherwise touch 32 rows at once). The running output rows of both
// blocks are loaded first, row-major; then per block the lanes of the MFMA
// layout stage O * cb and each row's (ca, write) pair, and the row-major
// lanes merge ca * old + staged and store. Rows whose previous lse is -inf
// take none of the loaded output (a select, not a product).
constexpr int kStageRow = 528;  // bytes per staged row: 128 floats + (ca, write) + pad

template <bool ACC, bool FIN>
__device__ __forceinline__ void epilogue_w64(const AttnArgs& a, const WorkItem& it, int qw0, int lane,
                                             floatx16 (&O0)[4], floatx16 (&O1)[4],
                                             const float (&m_run)[2], const float (&l_part)[2],
                                             unsigned char* stage) {
  constexpr int D = 128;
  const int n = lane & 31, hh = lane >> 5;
  if (qw0 >= a.Cq) return;  // the whole wave lies past the block
  const int rmax = a.Cq - 1 - qw0;  // last row of the wave inside the block
  const bool full = rmax >= 63;
  // wave-uniform bases at the wave's first row; per-lane 32-bit byte offsets
  unsigned char* ro = reinterpret_cast<unsigned char*>(a.run_out + it.b * a.ro_bs + it.h * a.ro_hs +
                                                       (int64_t)qw0 * D);
  float* rl = a.run_lse + it.b * a.rl_bs + it.h * a.rl_hs + qw0;
  unsigned char* fo = FIN ? reinterpret_cast<unsigned char*>(reinterpret_cast<__bf16*>(a.fin_out) +
                                                             it.b * a.fo_bs + it.h * a.fo_hs +
                                                             (int64_t)qw0 * D)
                          : nullptr;
  float* fl = FIN ? a.fin_lse + it.b * a.fl_bs + it.h * a.fl_hs + qw0 : nullptr;
  // row-major view: access i of block b is row 32b + 2i + hh, floats 4n .. 4n+3
  float4 old[2][16];
  float lse_old[2] = {-INFINITY, -INFINITY};
  if (ACC) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (32 * b + n <= rmax) lse_old[b] = rl[32 * b + n];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = min(32 * b + 2 * i + hh, rmax);
        old[b][i] = *reinterpret_cast<const float4*>(ro + (uint32_t)(r * D + 4 * n) * 4u);
      }
    }
  }
  // Merge factors of both blocks first, so their dependent chains overlap.
  // The row sum's two halves (lanes n and n + 32) meet through a lane swap;
  // the logarithms and exponentials are the hardware base-2 ones (about one
  // ulp; l >= 1 whenever the row saw a key, since the element that set the
  // reference contributed 1).
  constexpr float kLn2 = 0.693147180559945309f, kLog2e = 1.442695040888963407f;
  float lse_new[2], ca[2], cb[2];
  bool write[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part[b]),
                                                     __float_as_uint(l_part[b]), false, false);
    const float l = l_part[b] + __uint_as_float(hh ? sw[0] : sw[1]);
    const float m_use = (m_run[b] == -INFINITY) ? 0.f : m_run[b];
    const float lse_blk =
        (l > 0.f) ? fmaf(m_use, a.scale, __builtin_amdgcn_logf(l) * kLn2) : -INFINITY;
    write[b] = 32 * b + n <= rmax && !(ACC && !FIN && lse_blk == -INFINITY);
    const float mx = fmaxf(lse_old[b], lse_blk);
    if (mx == -INFINITY) {
      lse_new[b] = -INFINITY;
      ca[b] = 0.f;
      cb[b] = 0.f;
    } else {
      const float mn = fminf(lse_old[b], lse_blk);
      lse_new[b] = fmaf(__builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f((mn - mx) * kLog2e)),
                        kLn2, mx);
      ca[b] = (lse_old[b] == -INFINITY) ? 0.f
                                        : __builtin_amdgcn_exp2f((lse_old[b] - lse_new[b]) * kLog2e);
      cb[b] = (lse_blk == -INFINITY)
                  ? 0.f
                  : __builtin_amdgcn_exp2f((lse_blk - lse_new[b]) * kLog2e) * __builtin_amdgcn_rcpf(l);
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    floatx16(&O)[4] = b ? O1 : O0;
    // MFMA layout: lane (n, hh) holds d = 32T + 8g + 4hh + (0..3) of row n
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 r;
        r.x = O[T][4 * g4 + 0] * cb[b];
        r.y = O[T][4 * g4 + 1] * cb[b];
        r.z = O[T][4 * g4 + 2] * cb[b];
        r.w = O[T][4 * g4 + 3] * cb[b];
        *reinterpret_cast<float4*>(stage + n * kStageRow + (32 * T + 8 * g4 + 4 * hh) * 4) = r;
      }
    if (hh == 0) {
      *reinterpret_cast<float2*>(stage + n * kStageRow + 4 * D) = make_float2(ca[b], write[b] ? 1.f : 0.f);
      if (write[b]) (FIN ? fl : rl)[32 * b + n] = lse_new[b];
    }
#pragma unroll
    for (int i0 = 0; i0 < 16; i0 += 8) {
      // all LDS reads of 8 rows first, so they are in flight together
      float4 rs[8];
      float2 fs[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r_loc = 2 * (i0 + k) + hh;
        rs[k] = *reinterpret_cast<const float4*>(stage + r_loc * kStageRow + 16 * n);
        fs[k] = *reinterpret_cast<const float2*>(stage + r_loc * kStageRow + 4 * D);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k;
        const uint32_t e = (uint32_t)((32 * b + 2 * i + hh) * D + 4 * n);  // element offset
        float4 r = rs[k];
        if (ACC) {
          // rows left as they are (no key of the block) store their old value
          const bool use_old = fs[k].x != 0.f, keep = fs[k].y == 0.f;
          r.x = keep ? old[b][i].x : use_old ? fmaf(old[b][i].x, fs[k].x, r.x) : r.x;
          r.y = keep ? old[b][i].y : use_old ? fmaf(old[b][i].y, fs[k].x, r.y) : r.y;
          r.z = keep ? old[b][i].z : use_old ? fmaf(old[b][i].z, fs[k].x, r.z) : r.z;
          r.w = keep ? old[b][i].w : use_old ? fmaf(old[b][i].w, fs[k].x, r.w) : r.w;
        }
        // A wave whose 64 rows all lie in the block stores every row without
        // a branch; in the last, partial wave of a block rows past its end
        // are skipped.
        if (full || 32 * b + 2 * i + hh <= rmax) {
          if (FIN) {
            bf16x4 pk;
            pk[0] = (__bf16)r.x;
            pk[1] = (__bf16)r.y;
            pk[2] = (__bf16)r.z;
            pk[3] = (__bf16)r.w;
            *reinterpret_cast<bf16x4*>(fo + e * 2u) = pk;
          } else {
            *reinterpret_cast<float4*>(ro + e * 4u) = r;
          }
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------
// bf16 kernel: 64-key tiles, MFMA 32x32x16.
//
// Pipeline: K and V^T tiles are staged in two LDS buffers each by direct
// global->LDS loads. In iteration t a wave issues the score MFMAs of tile t+1
// with the softmax of tile t interleaved between them, then the P*V MFMAs of
// tile t (the two-group schedule below).
//
// Lazy rescale: the exponent reference m_run is not the running max. A tile's
// probabilities are computed against the current reference first; only if a
// lane's probabilities sum to more than 2^kRescaleLog2 (or it has no reference
// yet) is the true row max taken and the reference moved up. Probabilities are
// therefore bounded by 2^kRescaleLog2, the row max and the O^T rescale (64
// multiplies per lane) are skipped on almost every tile, and the result is
// unchanged, since l and O always share the same reference.
// ---------------------------------------------------------------------------
constexpr int kRescaleLog2 = 8;
constexpr float kFastSum = (float)(1 << kRescaleLog2);

// P*V operand stream of one 64-key tile: MFMA i (i = 0 .. 4*DT-1) takes
// u = i / DT (16-key step) and d tile T = i % DT; its V^T operand sits at
// byte offset T*32*VROW + u*32 from the lane's base address. Reads run PF
// ahead of the MFMAs in a ring of PF registers.
template <int D, int VROW>
struct PvStream {
  static constexpr int DT = D / 32, N = 4 * DT, PF = 4;
  static_assert(N >= PF, "fewer operands than reads in flight");
  static constexpr int off(int i) { return (i % DT) * 32 * VROW + (i / DT) * 32; }
  template <int I>
  static __device__ __forceinline__ void step(unsigned va, bf16x8 (&vr)[PF], floatx16 (&O)[DT],
                                              const bf16x8 (&P)[4]) {
    // reads issued after read I at this point: min(PF - 1, N - 1 - I)
    lds_wait<(N - 1 - I < PF - 1) ? (N - 1 - I) : (PF - 1)>(vr[I % PF]);
    O[I % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[I % PF], P[I / DT], O[I % DT], 0, 0, 0);
    if constexpr (I + PF < N) vr[I % PF] = ds_read16<off(I + PF)>(va);
    if constexpr (I + 1 < N) step<I + 1>(va, vr, O, P);
  }
  template <int I>
  static __device__ __forceinline__ void prefetch(unsigned va, bf16x8 (&vr)[PF]) {
    vr[I] = ds_read16<off(I)>(va);
    if constexpr (I + 1 < PF) prefetch<I + 1>(va, vr);
  }
  static __device__ __forceinline__ void run(unsigned va, floatx16 (&O)[DT], const bf16x8 (&P)[4]) {
    bf16x8 vr[PF];
    prefetch<0>(va, vr);
    step<0>(va, vr, O, P);
  }
};

struct QkNoWork {
  template <int I>
  __device__ __forceinline__ void operator()(std::integral_constant<int, I>) {}
};

// Score operand stream of one 64-key tile: 2*KS MFMAs alternating the two
// 32-key accumulators (MFMA i: key half i%2, k-step i/2; K operand at byte
// offset (i%2)*32*KROW + (i/2)*32 from the lane's base), operands read PF
// ahead through a register ring; after MFMA i the work functor gets step i.
template <int D, int KROW, int PF>
struct QkStream {
  static constexpr int KS = D / 16, N = 2 * KS;
  static constexpr int off(int i) { return (i % 2) * 32 * KROW + (i / 2) * 32; }
  template <int I, class W>
  static __device__ __forceinline__ void step(unsigned ka, bf16x8 (&r)[PF], const bf16x8 (&qreg)[KS],
                                              floatx16 (&S)[2], W& work) {
    lds_wait<(N - 1 - I < PF - 1) ? (N - 1 - I) : (PF - 1)>(r[I % PF]);
    S[I % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], qreg[I / 2], S[I % 2], 0, 0, 0);
    if constexpr (I + PF < N) r[I % PF] = ds_read16<off(I + PF)>(ka);
    work(std::integral_constant<int, I>{});
    if constexpr (I + 1 < N) step<I + 1>(ka, r, qreg, S, work);
  }
  template <int I>
  static __device__ __forceinline__ void prefetch(unsigned ka, bf16x8 (&r)[PF]) {
    r[I] = ds_read16<off(I)>(ka);
    if constexpr (I + 1 < PF) prefetch<I + 1>(ka, r);
  }
  template <class W>
  static __device__ __forceinline__ void run(unsigned ka, const bf16x8 (&qreg)[KS], floatx16 (&S)[2],
                                             W& work) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[t][i] = 0.f;
    bf16x8 r[PF];
    prefetch<0>(ka, r);
    step<0>(ka, r, qreg, S, work);
  }
};

// Probabilities of the current tile's 32 scores per lane, PER per score MFMA
// of the next tile: element e = 8u + j of P[u] is score Sc[u/2][8(u%2) + j].
template <int PER>
struct ProbsWork {
  const floatx16 (&Sc)[2];
  float c, moff;
  float (&rs)[4];
  bf16x8 (&P)[4];
  template <int I>
  __device__ __forceinline__ void operator()(std::integral_constant<int, I>) {
#pragma unroll
    for (int e = I * PER; e < (I + 1) * PER; ++e) {
      const int u = e >> 3, j = e & 7;
      const float p = __builtin_amdgcn_exp2f(fmaf(Sc[u >> 1][8 * (u & 1) + j], c, -moff));
      rs[u] += p;
      P[u][j] = (__bf16)p;
    }
    // the empty asm keeps this slice between its MFMAs: its values must
    // exist here, and volatile asm statements keep their order
    constexpr int ul = ((I + 1) * PER - 1) >> 3;
    asm volatile("" : "+v"(P[ul]), "+v"(rs[ul]));
  }
};

// Two-group schedule. A workgroup is 8 waves: group A (waves 0-3) and group B
// (waves 4-7), one wave of each on every SIMD. Each wave alternates
//   S-phase(t): softmax of tile t (VALU) and the score MFMAs of tile t+1,
//   P-phase(t): the P*V MFMAs of tile t,
// with a workgroup barrier after every phase; group B runs one barrier behind
// group A. On every SIMD both waves therefore issue LDS-fed MFMAs in every
// interval, and one of them also issues the softmax; that wave runs at raised
// issue priority. The direct tile loads are issued in the P-phases --
// group A loads V^T, group B loads K -- and drained before the barrier that
// ends the same wave's next S-phase; K and V^T each have two LDS buffers.
template <int D>
__global__ __launch_bounds__(kThreadsBf16, 1) void attn_fwd_bf16(const AttnArgs a) {
  constexpr int KS = D / 16;    // MFMA k-steps of the score product
  constexpr int DT = D / 32;    // 32-wide d tiles of the output
  constexpr int CPR = D / 8;             // 16-byte data chunks per K row
  constexpr int KCPR = CPR + 1;          // with the pad chunk
  constexpr int KROW = KCPR * 16;        // bytes per padded K row
  constexpr int VROW = 9 * 16;           // bytes per padded V^T row (64 keys + pad)
  constexpr int KBUF = 64 * KROW, VBUF = D * VROW;  // bytes per LDS tile
  constexpr int KINS = KBUF / 1024, VINS = VBUF / 1024;  // 1 KiB direct loads per tile
  constexpr int LW = 4;                  // waves per loading group (A: V^T, B: K)
  constexpr int KI = (KINS + LW - 1) / LW, VI = (VINS + LW - 1) / LW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* Ks = lds;             // [2][64 keys][D + 8]
  unsigned char* Vs = lds + 2 * KBUF;  // [2][D][64 + 8]

  WorkItem it;
  if (!decode_item(a, it)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grpB = wv >= 4;
  const int lw = wv & 3;
  const int n = lane & 31, hh = lane >> 5;
  const int qw0 = it.q0 + 32 * wv;
  const int qi = qw0 + n;
  const int qlast = a.Cq - 1;
  const int qpos = pos_of(a.qp, min(qi, qlast));
  const int wave_qmin = pos_of(a.qp, min(qw0, qlast));
  const int wg_qmax = pos_of(a.qp, min(it.q0 + a.q_tile - 1, qlast));
  const int n_keys = a.causal ? allowed_prefix(a.kp, wg_qmax) : a.Ck;
  const int n_kt = (n_keys + 63) / 64;
  const float c = a.scale_log2;

  const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + it.b * a.q_bs + it.h * a.q_hs;
  const __bf16* kbp = reinterpret_cast<const __bf16*>(a.k) + it.b * a.k_bs + it.g * a.k_hs;
  const __bf16* vtb = reinterpret_cast<const __bf16*>(a.v) + it.b * a.v_bs + it.g * a.v_hs;

  bf16x8 qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qi < a.Cq)
      qreg[s] = *reinterpret_cast<const bf16x8*>(qb + (int64_t)qi * D + 16 * s + 8 * hh);
    else
      for (int j = 0; j < 8; ++j) qreg[s][j] = (__bf16)0.f;
  }

  floatx16 O[DT];
#pragma unroll
  for (int T = 0; T < DT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[T][i] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;

  // Padded layouts: a K row is D+8 bf16 (CPR+1 chunks of 16 bytes), a V^T row
  // 64+8 bf16 (9 chunks). The 32 rows an MFMA operand read touches then fall
  // in distinct banks, and every operand offset is an immediate. A direct
  // load fills 64 consecutive chunks; lanes that land on a pad chunk re-read
  // a chunk of the same row.
  // Direct loads: instruction j of loading wave lw fills chunks
  // P = (lw + LW*j)*64 + lane of the tile (group B loads K, group A V^T).
  // Per-lane byte offsets of this wave's loads within a tile (K rows for
  // group B, V^T rows for group A), computed once: a full tile's load is then
  // a wave-uniform tile base plus one of these 32-bit offsets.
  constexpr int NL = KI > VI ? KI : VI;
  uint32_t loff[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int P = (lw + LW * j) * 64 + lane;
    if (grpB) {
      const int cch = P % KCPR;
      loff[j] = (uint32_t)((P / KCPR) * D + (cch < CPR ? cch : 0) * 8) * 2u;
    } else {
      const int cch = P % 9;
      loff[j] = ((uint32_t)(P / 9) * (uint32_t)a.v_ld + (uint32_t)(cch < 8 ? cch : 0) * 8u) * 2u;
    }
  }
  // the V^T offsets fit in 32 bits while a tile's D rows span < 4 GiB
  const bool v_off32 = (int64_t)D * a.v_ld * 2 <= (int64_t)UINT32_MAX;
  auto load_k = [&](int kt, int buf) {
    const int kb = kt * 64;
    unsigned char* dst = Ks + buf * KBUF + lw * 1024;
    if (kb + 64 <= a.Ck) {
      const unsigned char* base = reinterpret_cast<const unsigned char*>(kbp + (int64_t)kb * D);
#pragma unroll
      for (int j = 0; j < KI; ++j)
        if (lw + LW * j < KINS) load_lds16(base + loff[j], dst + j * LW * 1024);
      return;
    }
    // ragged last tile: rows past the block end re-read its last row (their
    // scores are masked)
    const int lane = lane_id();
    const int rows_left = a.Ck - 1 - kb;  // last valid row of this tile
    const __bf16* base = kbp + (int64_t)kb * D;
#pragma unroll
    for (int j = 0; j < KI; ++j)
      if (lw + LW * j < KINS) {
        const int P = (lw + LW * j) * 64 + lane;
        const int cch = P % KCPR;
        const int row = min(P / KCPR, rows_left);
        load_lds16(base + row * D + (cch < CPR ? cch : 0) * 8, dst + j * LW * 1024);
      }
  };
  auto load_v = [&](int kt, int buf) {
    unsigned char* dst = Vs + buf * VBUF + lw * 1024;
    if (v_off32) {
      const unsigned char* base = reinterpret_cast<const unsigned char*>(vtb + kt * 64);
#pragma unroll
      for (int j = 0; j < VI; ++j)
        if (lw + LW * j < VINS) load_lds16(base + loff[j], dst + j * LW * 1024);
      return;
    }
    const int lane = lane_id();
    const __bf16* base = vtb + kt * 64;
#pragma unroll
    for (int j = 0; j < VI; ++j)
      if (lw + LW * j < VINS) {
        const int P = (lw + LW * j) * 64 + lane;
        const int cch = P % 9;
        load_lds16(base + (int64_t)(P / 9) * a.v_ld + (cch < 8 ? cch : 0) * 8, dst + j * LW * 1024);
      }
  };

  // LDS read offsets of the MFMA operands (bytes, within one buffer).
  const int k_rbase = kperm(n) * KROW + hh * 16;  // + t*32*KROW + s*32
  const int v_rbase = n * VROW + hh * 16;         // + T*32*VROW + u*32

  // Score MFMAs of one tile through the K operand ring (four reads in
  // flight; the compiler's own schedule kept one or two and waited right
  // before the MFMA that needed it).
  using QK = QkStream<D, KROW, 4>;
  auto scores = [&](int kbuf, floatx16 (&S)[2]) {
    QkNoWork nw;
    QK::run(lds_addr(Ks) + kbuf * KBUF + k_rbase, qreg, S, nw);
  };
  // P*V of the tile in V buffer vbuf: 4*DT MFMAs (u-major, so the DT
  // accumulators alternate), each fed by one 16-byte V^T read, with reads kept
  // in flight in a register ring.
  auto pv_phase = [&](int vbuf, const bf16x8 (&P)[4]) {
    PvStream<D, VROW>::run(lds_addr(Vs) + vbuf * VBUF + v_rbase, O, P);
  };
  // Tiles that cross the causal diagonal or the ragged end of the block.
  auto needs_mask = [&](int kt) -> bool {
    const int kb = kt * 64;
    return kb + 64 > a.Ck || (a.causal && pos_of(a.kp, min(kb + 63, a.Ck - 1)) > wave_qmin);
  };
  auto apply_mask = [&](int kt, floatx16 (&Sc)[2]) {
    const int kb = kt * 64;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + 32 * t + 16 * (i >> 3) + 8 * hh + (i & 7);
        Sc[t][i] = masked(Sc[t][i], key, a.Ck, a.causal, a.kp, qpos);
      }
  };
  // Probabilities of scores Sc against the current reference m_run, into P
  // (bf16); returns this lane's fp32 sum of them (the unfused path: masked
  // tiles, the last tile, a rescale).
  auto probs = [&](const floatx16 (&Sc)[2], bf16x8 (&P)[4]) -> float {
    const float moff = (m_run == -INFINITY ? 0.f : m_run) * c;
    float rs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      rs[u] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(Sc[u >> 1][8 * (u & 1) + j], c, -moff));
        rs[u] += p;
        P[u][j] = (__bf16)p;
      }
    }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };
  // Fast path: a reference exists and this lane's probabilities sum to at
  // most 2^kRescaleLog2, so none exceeds it -- no row max is needed.
  // Otherwise take the row max and move the reference where it grew.
  auto finish = [&](const floatx16 (&Sc)[2], bf16x8 (&P)[4], float rsum) {
    const bool slow = !(rsum <= kFastSum) || (m_run == -INFINITY);
    if (__any(slow)) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, Sc[t][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool grow = mx > m_run;
      if (__any(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.f;
#pragma unroll
        for (int T = 0; T < DT; ++T)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[T][i] *= alpha;
        l_part *= alpha;
        m_run = m_new;
        rsum = probs(Sc, P);
      }
    }
    l_part += rsum;
  };
  // Scores of the next tile (K buffer kbuf) into Sn, interleaved with the
  // probabilities of the current unmasked tile Sc: each score MFMA is
  // followed by a slice of the softmax arithmetic (the stream's work
  // functor), so the exp/fma/add stream runs under this wave's own matrix
  // work.
  auto scores_probs = [&](int kbuf, floatx16 (&Sn)[2], const floatx16 (&Sc)[2],
                          bf16x8 (&P)[4]) -> float {
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    ProbsWork<32 / QK::N> w{Sc, c, (m_run == -INFINITY ? 0.f : m_run) * c, rs, P};
    QK::run(lds_addr(Ks) + kbuf * KBUF + k_rbase, qreg, Sn, w);
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };

  if (n_kt > 0) {
    floatx16 SA[2], SB[2];
    bf16x8 P[4];
    // prologue: K0, K1 (group B) and V0 (group A) in LDS; every wave takes
    // the scores of tile 0; group B then loads K2 and falls one barrier behind.
    if (grpB) {
      load_k(0, 0);
      if (n_kt > 1) load_k(1, 1);
    } else {
      load_v(0, 0);
    }
    lds_loads_barrier();
    scores(0, SA);
    __syncthreads();  // every wave is done with K0
    if (grpB) {
      if (n_kt > 2) load_k(2, 0);
      lds_loads_barrier();
    }
    // S-phase(t) / P-phase(t); Sc holds the scores of tile t, Sn receives
    // those of tile t+1.
    auto tile = [&](int t, floatx16 (&Sc)[2], floatx16 (&Sn)[2]) {
      // The S-phase wave (MFMAs plus the softmax VALU stream) is the longer
      // of the two on a SIMD; raising its issue priority lets the P-phase
      // wave's MFMAs fill the matrix pipe around it instead of delaying it.
      __builtin_amdgcn_s_setprio(1);
      float rsum;
      if (t + 1 < n_kt && !needs_mask(t)) {
        rsum = scores_probs((t + 1) & 1, Sn, Sc, P);
      } else {
        if (t + 1 < n_kt) scores((t + 1) & 1, Sn);
        if (needs_mask(t)) apply_mask(t, Sc);
        rsum = probs(Sc, P);
      }
      finish(Sc, P, rsum);
      __builtin_amdgcn_s_setprio(0);
      // this wave's loads from its last P-phase land before the barrier
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      workgroup_barrier();
      if (grpB) {
        if (t + 3 < n_kt) load_k(t + 3, (t + 1) & 1);
      } else {
        if (t + 1 < n_kt) load_v(t + 1, (t + 1) & 1);
      }
      pv_phase(t & 1, P);
      workgroup_barrier();
    };
    int t = 0;
    for (; t + 1 < n_kt; t += 2) {
      tile(t, SA, SB);
      tile(t + 1, SB, SA);
    }
    if (t < n_kt) tile(t, SA, SB);
    if (!grpB) __syncthreads();  // group A matches group B's extra barrier
  }
  epilogue<DT, true>(a, it, qi, hh, O, m_run, l_part);
}

// LDS bytes of the bf16 kernel (two padded K and two padded V^T tiles).
constexpr size_t bf16_lds_bytes(int D) { return (size_t)2 * (64 * (D / 8 + 1) * 16 + D * 9 * 16); }
// K tiles in w64::kKBufs buffers, V^T tiles in two, and a 64-row staging
// area per wave (D = 128).
constexpr size_t w64_lds_bytes() {
  return (size_t)(w64::kKBufs + 4) * 64 * 17 * 16 + 2 * 128 * 9 * 16;
}

// ---------------------------------------------------------------------------
// bf16 kernel for D = 128, one wave per SIMD: 4 waves x 64 query rows (two
// 32-row blocks per wave). Every K or V^T operand read from LDS feeds two
// MFMAs, one per row block, and the wave's own instruction stream overlaps
// its matrix and vector work:
//   phase A(t): score MFMAs of tile t+1 (both blocks) with the softmax of
//               block 1 of tile t between them;
//   phase B(t): P*V MFMAs of tile t (both blocks) with the softmax of
//               block 0 of tile t+1 between them.
// The whole key loop -- both phases, the masks, the lazy-rescale check and
// the tile loads -- is one inline-asm statement with a fixed schedule and
// fixed registers (attn_fwd_w64_phases.h, written by gen_fwd_w64.py). K tiles
// rotate through three LDS buffers and V^T tiles through two; all four waves
// load both, and one barrier per tile publishes the loads and frees the
// buffers they refill. Around the loop, each wave stages its query rows and
// its output rows through an LDS area of its own, so that the state in
// global memory is read and written in whole rows.
// ---------------------------------------------------------------------------
constexpr int kWavesW64 = 4;
constexpr int kThreadsW64 = 64 * kWavesW64;

__global__ __launch_bounds__(kThreadsW64, 1) void attn_fwd_bf16_w64(const AttnArgs a) {
  constexpr int D = 128;
  constexpr int KS = D / 16;             // MFMA k-steps of the score product
  constexpr int DT = D / 32;             // 32-wide d tiles of the output
  constexpr int CPR = D / 8;             // 16-byte data chunks per K row
  constexpr int KCPR = CPR + 1;          // with the pad chunk
  constexpr int KROW = KCPR * 16;        // bytes per padded K row
  constexpr int VROW = 9 * 16;           // bytes per padded V^T row (64 keys + pad)
  constexpr int KBUF = 64 * KROW, VBUF = D * VROW;  // bytes per LDS tile
  constexpr int KINS = KBUF / 1024, VINS = VBUF / 1024;  // 1 KiB direct loads per tile
  constexpr int NW = kWavesW64;
  constexpr int KI = (KINS + NW - 1) / NW, VI = (VINS + NW - 1) / NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* Ks = lds;                           // [kKBufs][64 keys][D + 8]
  unsigned char* Vs = lds + w64::kKBufs * KBUF;      // [2][D][64 + 8]
  // per wave: its 64 query rows (padded like K) in the prologue, its output
  // rows on the way out
  unsigned char* Stage = Vs + 2 * VBUF;              // [NW][64 rows][D + 8]
  static_assert(32 * kStageRow <= KBUF, "a staged 32-row block fits a wave's area");
  static_assert(NW == 4 && w64_lds_bytes() == (size_t)(w64::kKBufs + NW) * KBUF + 2 * VBUF &&
                    w64_lds_bytes() <= 160 * 1024,
                "LDS layout of the one-wave-per-SIMD kernel");

  WorkItem it;
  if (!decode_item(a, it)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int qlast = a.Cq - 1;
  const int qw0 = it.q0 + 64 * wv;                 // first row of the wave
  const int qi0 = qw0 + n, qi1 = qw0 + 32 + n;     // this lane's row in block 0 / 1

  const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + it.b * a.q_bs + it.h * a.q_hs;
  const __bf16* kbp = reinterpret_cast<const __bf16*>(a.k) + it.b * a.k_bs + it.g * a.k_hs;
  const __bf16* vtb = reinterpret_cast<const __bf16*>(a.v) + it.b * a.v_bs + it.g * a.v_hs;

  // Per-lane byte offsets of this wave's prologue loads within a K tile and
  // a V^T tile (instruction j fills 1 KiB chunk wv + NW*j of the tile).
  // The tail chunks of a tile (K: 17 KiB, V^T: 18 KiB) go to different waves
  // (K to wave 0, V^T to waves 2 and 3), so no wave issues more than nine
  // loads per tile: V^T chunks are dealt starting from wave 2.
  const int vw = (wv + 2) % NW;
  uint32_t koff[KI], voff[VI];
#pragma unroll
  for (int j = 0; j < KI; ++j) {
    const int P = (wv + NW * j) * 64 + lane;
    const int cch = P % KCPR;
    koff[j] = (uint32_t)((P / KCPR) * D + (cch < CPR ? cch : 0) * 8) * 2u;
  }
#pragma unroll
  for (int j = 0; j < VI; ++j) {
    const int P = (vw + NW * j) * 64 + lane;
    const int cch = P % 9;
    voff[j] = ((uint32_t)(P / 9) * (uint32_t)a.v_ld + (uint32_t)(cch < 8 ? cch : 0) * 8u) * 2u;
  }
  // Whole tiles only (the block is a multiple of 64 keys and the V^T rows of
  // a tile lie within 4 GiB: the launch dispatches other blocks to the
  // 8-wave kernel), so every load is a tile base plus a 32-bit offset.
  auto load_k = [&](int kt, int buf) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(kbp + (int64_t)kt * 64 * D);
    unsigned char* dst = Ks + buf * KBUF + wv * 1024;
#pragma unroll
    for (int j = 0; j < KI; ++j)
      if (wv + NW * j < KINS) load_lds16(base + koff[j], dst + j * NW * 1024);
  };
  auto load_v = [&](int kt, int buf) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(vtb + kt * 64);
    unsigned char* dst = Vs + buf * VBUF + vw * 1024;
#pragma unroll
    for (int j = 0; j < VI; ++j)
      if (vw + NW * j < VINS) load_lds16(base + voff[j], dst + j * NW * 1024);
  };

  // Prologue loads, issued before anything else is worked out: the wave's
  // query rows (whole-row loads into its staging area; the pad chunk repeats
  // chunk 0, rows past the block repeat the last one), the first kKBufs K
  // tiles of the block and V^T tile 0, of those the block has. Tiles the
  // causal mask leaves unused are loaded all the same (they lie inside the
  // block).
  unsigned char* stage = Stage + wv * KBUF;
  {
    const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(qb);
#pragma unroll
    for (int j = 0; j < KCPR; ++j) {
      const int P = j * 64 + lane, cch = P % KCPR;
      const int row = min(qw0 + P / KCPR, qlast);
      load_lds16(qbytes + ((int64_t)row * D + (cch < CPR ? cch : 0) * 8) * 2, stage + j * 1024);
    }
#pragma unroll
    for (int j = 0; j < w64::kKBufs; ++j)
      if (64 * j < a.Ck) load_k(j, j);
    if (a.Ck > 0) load_v(0, 0);  // an empty block has no V^T tile
  }

  // Keys of the block each row may see (a prefix: positions increase along
  // the block); tiles before first_mask are fully visible to every row of
  // the wave, later ones are masked per lane.
  const int qpos0 = pos_of(a.qp, min(qi0, qlast));
  const int qpos1 = pos_of(a.qp, min(qi1, qlast));
  const int wave_qmin = pos_of(a.qp, min(qw0, qlast));
  const int wg_qmax = pos_of(a.qp, min(it.q0 + a.q_tile - 1, qlast));
  const int n_keys = a.causal ? allowed_prefix(a.kp, wg_qmax) : a.Ck;
  const int n_kt = (n_keys + 63) / 64;
  const int nal0 = a.causal ? allowed_prefix(a.kp, qpos0) : a.Ck;
  const int nal1 = a.causal ? allowed_prefix(a.kp, qpos1) : a.Ck;
  const int first_mask = a.causal ? allowed_prefix(a.kp, wave_qmin) / 64 : n_kt;
  const float c = a.scale_log2;

  floatx16 O0[DT], O1[DT];
  float m0 = -INFINITY, l0 = 0.f, m1 = -INFINITY, l1 = 0.f;
  lds_loads_barrier();  // also when no tile is needed: no load may outlive the workgroup
  if (n_kt > 0) {
    bf16x8 q0[KS], q1[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      q0[s] = *reinterpret_cast<const bf16x8*>(stage + n * KROW + 32 * s + 16 * hh);
      q1[s] = *reinterpret_cast<const bf16x8*>(stage + (n + 32) * KROW + 32 * s + 16 * hh);
      if (qi0 >= a.Cq)
        for (int j = 0; j < 8; ++j) q0[s][j] = (__bf16)0.f;
      if (qi1 >= a.Cq)
        for (int j = 0; j < 8; ++j) q1[s][j] = (__bf16)0.f;
    }
    // wave-uniform values the loop keeps in SGPRs
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    auto uni_ptr = [](const void* p) {
      const uint64_t v = (uint64_t)(size_t)p;
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      return (const void*)(size_t)(((uint64_t)hi << 32) | lo);
    };
    // In the loop every wave loads five contiguous chunks of each tile, from
    // chunk kc0 of a K tile (17 chunks) and vc0 of a V^T tile (18); the
    // ranges overlap on a few chunks, which two waves load with the same
    // data. The loop places the five loads from M0 = the wave's last chunk
    // with instruction offsets -4 KiB .. 0, which move the global address
    // too: the lane offsets carry the opposite amount.
    static_assert(KI == 5 && VI == 5 && KINS == 17 && VINS == 18, "five chunk loads per tile");
    const int kc0 = wv == 0 ? 0 : wv == 1 ? 4 : wv == 2 ? 8 : 12;
    const int vc0 = wv == 0 ? 0 : wv == 1 ? 4 : wv == 2 ? 9 : 13;
    uint32_t koffa[KI], voffa[VI];
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const int P = (kc0 + j) * 64 + lane, cch = P % KCPR;
      koffa[j] = (uint32_t)((P / KCPR) * D + (cch < CPR ? cch : 0) * 8) * 2u + (uint32_t)(4 - j) * 1024u;
    }
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const int P = (vc0 + j) * 64 + lane, cch = P % 9;
      voffa[j] = ((uint32_t)(P / 9) * (uint32_t)a.v_ld + (uint32_t)(cch < 8 ? cch : 0) * 8u) * 2u +
                 (uint32_t)(4 - j) * 1024u;
    }
    w64::attn_loop(uni(n_kt), uni(first_mask), uni(lds_addr(Ks) + (kc0 + 4) * 1024),
                   uni(lds_addr(Vs) + (vc0 + 4) * 1024), c,
                   lds_addr(Ks) + kperm(n) * KROW + hh * 16, lds_addr(Vs) + n * VROW + hh * 16,
                   nal0 - 8 * hh, nal1 - 8 * hh, (unsigned)((lane ^ 32) * 4),
                   uni_ptr(kbp + (int64_t)min(w64::kKBufs, n_kt - 1) * 64 * D), uni_ptr(vtb + 64), koffa, voffa,
                   q0, q1, O0, O1, m0, l0, m1, l1);
  } else {
#pragma unroll
    for (int T = 0; T < DT; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        O0[T][i] = 0.f;
        O1[T][i] = 0.f;
      }
  }
  const float ms[2] = {m0, m1}, ls[2] = {l0, l1};
  if (a.fin_out) {
    if (a.accumulate)
      epilogue_w64<true, true>(a, it, qw0, lane, O0, O1, ms, ls, stage);
    else
      epilogue_w64<false, true>(a, it, qw0, lane, O0, O1, ms, ls, stage);
  } else {
    if (a.accumulate)
      epilogue_w64<true, false>(a, it, qw0, lane, O0, O1, ms, ls, stage);
    else
      epilogue_w64<false, false>(a, it, qw0, lane, O0, O1, ms, ls, stage);
  }
}


// ---------------------------------------------------------------------------
// fp32 kernel: 32-key tiles, MFMA 32x32x2 f32, V row-major.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_f32(const AttnArgs a) {
  constexpr int KS = D / 2;
  constexpr int DT = D / 32;
  constexpr int KLD = D + 1;
  constexpr int VLD = D + 4;
  constexpr int CH = 32 * D / 4 / kThreads;  // float4 chunks per thread per tile
  __shared__ __attribute__((aligned(16))) float Ks[32 * KLD];
  __shared__ __attribute__((aligned(16))) float Vs[32 * VLD];

  WorkItem it;
  if (!decode_item(a, it)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int qw0 = it.q0 + 32 * wv;
  const int qi = qw0 + n;
  const int qlast = a.Cq - 1;
  const int qpos = pos_of(a.qp, min(qi, qlast));
  const int wave_qmin = pos_of(a.qp, min(qw0, qlast));
  const int wg_qmax = pos_of(a.qp, min(it.q0 + a.q_tile - 1, qlast));
  const int n_keys = a.causal ? allowed_prefix(a.kp, wg_qmax) : a.Ck;
  const int n_kt = (n_keys + 31) / 32;

  const float* qb = reinterpret_cast<const float*>(a.q) + it.b * a.q_bs + it.h * a.q_hs;
  const float* kbp = reinterpret_cast<const float*>(a.k) + it.b * a.k_bs + it.g * a.k_hs;
  const float* vbp = reinterpret_cast<const float*>(a.v) + it.b * a.v_bs + it.g * a.v_hs;

  float qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qreg[s] = (qi < a.Cq) ? qb[(int64_t)qi * D + 2 * s + hh] : 0.f;

  floatx16 O[DT];
#pragma unroll
  for (int T = 0; T < DT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[T][i] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;

  float4 kreg[CH], vreg[CH];
  auto load_tile = [&](int kt) {
    const int kb = kt * 32;
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 4), col = c % (D / 4);
      const int key = kb + row;
      if (key < a.Ck) {
        kreg[r] = *reinterpret_cast<const float4*>(kbp + (int64_t)key * D + col * 4);
        vreg[r] = *reinterpret_cast<const float4*>(vbp + (int64_t)key * D + col * 4);
      } else {
        kreg[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        vreg[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 4), col = c % (D / 4);
      float* kd = &Ks[row * KLD + col * 4];
      kd[0] = kreg[r].x;
      kd[1] = kreg[r].y;
      kd[2] = kreg[r].z;
      kd[3] = kreg[r].w;
      *reinterpret_cast<float4*>(&Vs[row * VLD + col * 4]) = vreg[r];
    }
  };

  if (n_kt > 0) load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);

    floatx16 S[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) S[0][i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[n * KLD + 2 * s + hh], qreg[s], S[0], 0, 0,
                                                   0);

    // Lane (n, hh), register i holds key kb + 4*hh + (i%4) + 8*(i/4).
    const int kb = kt * 32;
    const bool ragged = kb + 32 > a.Ck;
    const bool diag = a.causal && pos_of(a.kp, min(kb + 31, a.Ck - 1)) > wave_qmin;
    if (ragged || diag) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + 4 * hh + (i & 3) + 8 * (i >> 2);
        S[0][i] = masked(S[0][i], key, a.Ck, a.causal, a.kp, qpos);
      }
    }

    const float alpha = softmax_tile<1>(S, m_run, l_part, a.scale_log2);
#pragma unroll
    for (int T = 0; T < DT; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[T][i] *= alpha;

#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int krow = 4 * hh + (i & 3) + 8 * (i >> 2);
#pragma unroll
      for (int T = 0; T < DT; ++T)
        O[T] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[krow * VLD + 32 * T + n], S[0][i], O[T],
                                                     0, 0, 0);
    }
  }
  epilogue<DT, false>(a, it, qi, hh, O, m_run, l_part);
}

}  // namespace

// ---------------------------------------------------------------------------
// Host-side work list.
// ---------------------------------------------------------------------------
namespace {
inline int64_t floordiv_i64(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// First row of a block whose position is >= P (rows if none).
int64_t first_row_at_or_after(const PosDesc& p, int64_t rows, int64_t P) {
  const int64_t seg0 = p.nseg == 2 ? p.seg : rows;
  const int64_t last0 = (int64_t)p.start0 + (seg0 - 1) * p.stride;
  if (P <= last0) return std::max<int64_t>(0, -floordiv_i64(-(P - p.start0), p.stride));
  if (p.nseg == 2 && P <= (int64_t)p.start1 + (int64_t)(p.seg - 1) * p.stride)
    return p.seg + std::max<int64_t>(0, -floordiv_i64(-(P - p.start1), p.stride));
  return rows;
}

}  // namespace

void fill_attn_work(AttnArgs& a, ra_dtype dt, int32_t B, int32_t Hq, int64_t Cq,
                    const std::vector<uint8_t>& kv_of, const std::vector<uint8_t>& order) {
  memset(a.head_order, 0, sizeof a.head_order);
  memset(a.kv_of, 0, sizeof a.kv_of);
  for (int h = 0; h < Hq; ++h) {
    a.head_order[h] = order[h];
    a.kv_of[h] = kv_of[h];
  }
  a.B = B;
  a.Hq = Hq;
  const int32_t qtile = dt == RA_BF16 ? kQTileBf16 : kQTileF32;
  a.q_tile = qtile;
  const int32_t n_qt_all = (int32_t)((Cq + qtile - 1) / qtile);
  // With accumulate = 1, leading query tiles that see no key are skipped:
  // positions increase with the row index, so these are the rows whose
  // position is below the block's first key position. Not on the final step
  // of the ring, where every row still has to be written out.
  int32_t lo = 0;
  if (a.causal && a.accumulate && a.fin_out == nullptr) {
    const int64_t row = a.Ck > 0 ? first_row_at_or_after(a.qp, Cq, a.kp.start0) : Cq;
    lo = (int32_t)(row / qtile);
  }
  a.qt_lo = lo;
  a.n_qt = n_qt_all - lo;
  const int64_t items = (int64_t)B * Hq * a.n_qt;
  a.n_items = (int32_t)items;
  a.per_xcd = (int32_t)((items + kXcds - 1) / kXcds);
}

hipError_t launch_attn(const AttnArgs& a, ra_dtype dt, int D, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid((unsigned)(a.per_xcd * kXcds)), block(kThreads);
  if (dt == RA_BF16) {
    // The dynamic-LDS limit is a per-device property of the function: set it
    // on every launch (a host-side call), so any device and any thread that
    // launches through the library has it.
    // D = 128 blocks of whole 64-key tiles run on the one-wave-per-SIMD
    // kernel; ragged blocks, V^T rows more than 4 GiB apart and D = 64 on
    // the 8-wave kernel.
    const bool w64 = D == 128 && a.Ck % 64 == 0 && (int64_t)D * a.v_ld * 2 <= (int64_t)UINT32_MAX;
    const void* fn = w64 ? (const void*)attn_fwd_bf16_w64
                         : (D == 128 ? (const void*)attn_fwd_bf16<128> : (const void*)attn_fwd_bf16<64>);
    const size_t lds = w64 ? w64_lds_bytes() : bf16_lds_bytes(D);
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (w64)
      hipLaunchKernelGGL(attn_fwd_bf16_w64, grid, dim3(kThreadsW64), lds, s, a);
    else if (D == 128)
      hipLaunchKernelGGL(attn_fwd_bf16<128>, grid, dim3(kThreadsBf16), lds, s, a);
    else
      hipLaunchKernelGGL(attn_fwd_bf16<64>, grid, dim3(kThreadsBf16), lds, s, a);
  } else {
    if (D == 128)
      hipLaunchKernelGGL(attn_fwd_f32<128>, grid, block, 0, s, a);
    else
      hipLaunchKernelGGL(attn_fwd_f32<64>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ra
