// Backward of blockwise attention for one (query block, key block) pair -- the
// per-step kernels of the ring-attention backward pass.
//
// Method: the gradients are those of exact softmax attention ("Sequence and
// Context Parallelism", section "What it does not change"); the attention
// probabilities are recomputed from the saved log-sum-exp rather than stored
// ("Sequence Parallelism in Large Language Models ...", section "The
// Activation Memory Wall"); the ring schedule is the forward's ("Algorithmic
// Mechanics"). With p = exp(scale*q.k - lse) on allowed pairs, delta = <dout,
// out> per query row and ds = p (dp - delta), dp = <dout, v>:
//   dv_j = sum_i p_ij dout_i,  dk_j = scale sum_i ds_ij q_i,  dq_i = scale sum_j ds_ij k_j.
//
// gfx950 design (bf16 inputs, fp32 accumulation, v_mfma_f32_32x32x16_bf16):
//  * attn_bwd_dkdv: a workgroup owns 128 keys of one KV head (a wave owns 32,
//    its K and V rows in registers) and walks the query tiles (64 rows) of
//    every query head that reads the KV head. S = Q K^T and dP = dO V^T are
//    computed with the query rows permuted (kperm), so a lane holds the 16
//    queries of one key that the next MFMAs need as 8-query B operands:
//    dV^T += dO^T P and dK^T += Q^T dS, with Q^T and dO^T tiles in LDS.
//  * attn_bwd_dq: a workgroup owns 128 queries of one query head (Q and dO
//    rows of a wave in registers, as in the forward) and walks the key tiles
//    (64 keys): S^T = K Q^T and dP^T = V dO^T with kperm'd key rows, then
//    dQ^T += K^T dS^T with a K^T tile in LDS.
//  * All tiles move global->LDS with direct 16-byte loads into padded rows
//    (bank-conflict-free operand reads), double buffered, one barrier per
//    tile. Both kernels add into fp32 accumulators, so the ring can sum the
//    contributions of all block pairs.
#include "attn_common.h"

namespace ra {
namespace {

template <int D>
struct BwdLds {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row of D bf16
  static constexpr int RCPR = CPR + 1;          // with the pad chunk
  static constexpr int ROW = RCPR * 16;         // padded row of D bf16
  static constexpr int TROW = 9 * 16;           // padded row of 64 bf16 (transposed tiles)
  static constexpr int RBUF = 64 * ROW;         // 64 rows
  static constexpr int TBUF = D * TROW;         // D rows of 64
  static constexpr int RINS = RBUF / 1024;      // 1 KiB direct loads per row tile
  static constexpr int TINS = TBUF / 1024;      // ... per transposed tile
  static_assert(RBUF % 1024 == 0 && TBUF % 1024 == 0, "tiles are whole 1 KiB loads");
};

// Rows [0, 64) of a row-major [rows][D] tile into padded LDS rows; rows past
// rows_left re-read row rows_left (their contributions are masked or unused).
template <int D>
__device__ __forceinline__ void load_row_tile(const __bf16* base, int rows_left, unsigned char* dst,
                                              int wv, int lane) {
  using L = BwdLds<D>;
#pragma unroll
  for (int j = 0; j < (L::RINS + 3) / 4; ++j) {
    const int ins = wv + 4 * j;
    if (ins < L::RINS) {
      const int P = ins * 64 + lane;
      const int cch = P % L::RCPR;
      const int row = min(P / L::RCPR, rows_left);
      load_lds16(base + (int64_t)row * D + (cch < L::CPR ? cch : 0) * 8, dst + ins * 1024);
    }
  }
}

// Columns [0, 64) of a transposed [D][ld] array into padded LDS rows.
template <int D>
__device__ __forceinline__ void load_trans_tile(const __bf16* base, int64_t ld, unsigned char* dst,
                                                int wv, int lane) {
  using L = BwdLds<D>;
#pragma unroll
  for (int j = 0; j < (L::TINS + 3) / 4; ++j) {
    const int ins = wv + 4 * j;
    if (ins < L::TINS) {
      const int P = ins * 64 + lane;
      const int cch = P % 9;
      load_lds16(base + (P / 9) * ld + (cch < 8 ? cch : 0) * 8, dst + ins * 1024);
    }
  }
}

__device__ __forceinline__ int xcd_item(int n_items, int per_xcd) {
  const int w = blockIdx.x;
  const int L = (w % kXcds) * per_xcd + (w / kXcds);
  return L < n_items ? L : -1;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 4 waves x 32 keys of one KV head.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv(const BwdArgs a) {
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int OFF_DO = L::RBUF, OFF_QT = 2 * L::RBUF, OFF_DOT = 2 * L::RBUF + L::TBUF;
  constexpr int OFF_L = 2 * L::RBUF + 2 * L::TBUF, OFF_DL = OFF_L + 256, BUF = OFF_DL + 256;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int item = xcd_item(a.n_items, a.per_xcd);
  if (item < 0) return;
  const int kt = item % a.n_tiles;
  const int rest = item / a.n_tiles;
  const int g = rest % a.Hkv, b = rest / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int k0 = kt * 128, kw0 = k0 + 32 * wv;
  const int keyc = min(kw0 + n, a.Ck - 1);
  const float c = a.scale_log2;

  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k) + b * a.k_bs + g * a.k_hs;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v) + b * a.k_bs + g * a.k_hs;
  bf16x8 kreg[KS], vreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kreg[s] = *reinterpret_cast<const bf16x8*>(kbase + (int64_t)keyc * D + 16 * s + 8 * hh);
    vreg[s] = *reinterpret_cast<const bf16x8*>(vbase + (int64_t)keyc * D + 16 * s + 8 * hh);
  }
  floatx16 dKt[DT], dVt[DT];
#pragma unroll
  for (int T = 0; T < DT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dKt[T][i] = 0.f;
      dVt[T][i] = 0.f;
    }
  const int kpos = pos_of(a.kp, keyc);
  const int wave_kmax = pos_of(a.kp, min(kw0 + 31, a.Ck - 1));
  const int wg_kmin = pos_of(a.kp, min(k0, a.Ck - 1));
  // query rows before the first one that sees a key of this workgroup
  const int q_lo = a.causal ? allowed_prefix(a.qp, wg_kmin - 1) : 0;
  const int t_lo = q_lo / 64;
  const int n_t = max(0, (a.Cq + 63) / 64 - t_lo);
  const int rbase = kperm(n) * L::ROW + hh * 16;  // A operand of S / dP (+32 rows per sub-tile)

  for (int gi = a.grp_off[g]; gi < a.grp_off[g + 1]; ++gi) {
    const int h = a.head_order[gi];
    const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + b * a.q_bs + h * a.q_hs;
    const __bf16* db = reinterpret_cast<const __bf16*>(a.dout) + b * a.q_bs + h * a.q_hs;
    const __bf16* qtb = reinterpret_cast<const __bf16*>(a.qt) + b * a.qt_bs + h * a.qt_hs;
    const __bf16* dtb = reinterpret_cast<const __bf16*>(a.dot) + b * a.qt_bs + h * a.qt_hs;
    const float* l2b = a.lse2 + b * a.l_bs + h * a.l_hs;
    const float* dlb = a.delta + b * a.l_bs + h * a.l_hs;
    auto load_tile = [&](int t, int buf) {
      const int q0 = (t_lo + t) * 64;
      unsigned char* B0 = lds + buf * BUF;
      load_row_tile<D>(qb + (int64_t)q0 * D, a.Cq - 1 - q0, B0, wv, lane);
      load_row_tile<D>(db + (int64_t)q0 * D, a.Cq - 1 - q0, B0 + OFF_DO, wv, lane);
      load_trans_tile<D>(qtb + q0, a.Cqp, B0 + OFF_QT, wv, lane);
      load_trans_tile<D>(dtb + q0, a.Cqp, B0 + OFF_DOT, wv, lane);
      if (wv == 0 && lane < 16) load_lds16(l2b + q0 + 4 * lane, B0 + OFF_L);
      if (wv == 1 && lane < 16) load_lds16(dlb + q0 + 4 * lane, B0 + OFF_DL);
    };
    if (n_t > 0) load_tile(0, 0);
    for (int t = 0; t < n_t; ++t) {
      lds_loads_barrier();  // tile t landed; every wave is done with tile t-1
      if (t + 1 < n_t) load_tile(t + 1, (t + 1) & 1);
      const unsigned char* B0 = lds + (t & 1) * BUF;
      const int q0 = (t_lo + t) * 64;
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys;
        // element i of a lane is query 32qs + 16(i/8) + 8hh + i%8 of the tile
        floatx16 S, dP;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          S[i] = 0.f;
          dP[i] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(B0 + rbase + qs * 32 * L::ROW + s * 32);
          const bf16x8 da =
              *reinterpret_cast<const bf16x8*>(B0 + OFF_DO + rbase + qs * 32 * L::ROW + s * 32);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[s], S, 0, 0, 0);
          dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vreg[s], dP, 0, 0, 0);
        }
        const int qrow0 = q0 + 32 * qs;
        const bool need_mask = a.causal && pos_of(a.qp, min(qrow0, a.Cq - 1)) < wave_kmax;
        bf16x8 Pb[2], dSb[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int r0 = 32 * qs + 16 * w + 8 * hh;  // first of this lane's 8 rows
          const float* lp = reinterpret_cast<const float*>(B0 + OFF_L) + r0;
          const float* dp_ = reinterpret_cast<const float*>(B0 + OFF_DL) + r0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * w + j;
            float sc = S[i] * c - lp[j];
            if (need_mask) {
              const int qp_ = pos_of(a.qp, min(q0 + r0 + j, a.Cq - 1));
              sc = (kpos <= qp_) ? sc : -INFINITY;
            }
            const float p = __builtin_amdgcn_exp2f(sc);
            Pb[w][j] = (__bf16)p;
            dSb[w][j] = (__bf16)(p * (dP[i] - dp_[j]));
          }
        }
        // dV^T += dO^T P, dK^T += Q^T dS (A: row d of the transposed tiles)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int T = 0; T < DT; ++T) {
            const int toff = (32 * T + n) * L::TROW + (32 * qs + 16 * u + 8 * hh) * 2;
            const bf16x8 doa = *reinterpret_cast<const bf16x8*>(B0 + OFF_DOT + toff);
            const bf16x8 qta = *reinterpret_cast<const bf16x8*>(B0 + OFF_QT + toff);
            dVt[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(doa, Pb[u], dVt[T], 0, 0, 0);
            dKt[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, dSb[u], dKt[T], 0, 0, 0);
          }
      }
    }
    __syncthreads();  // the next head's first tile reuses buffer 0
  }

  // epilogue: add into the fp32 accumulators; lane holds key kw0+n,
  // d = 32T + 8(i/4) + 4hh + i%4
  const int key = kw0 + n;
  if (key < a.Ck) {
    float* dkr = a.dk + b * a.dk_bs + g * a.dk_hs + (int64_t)key * D;
    float* dvr = a.dv + b * a.dk_bs + g * a.dk_hs + (int64_t)key * D;
#pragma unroll
    for (int T = 0; T < DT; ++T)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * T + 8 * q4 + 4 * hh;
        float4 k4 = *reinterpret_cast<float4*>(dkr + d0);
        float4 v4 = *reinterpret_cast<float4*>(dvr + d0);
        k4.x += a.scale * dKt[T][4 * q4 + 0];
        k4.y += a.scale * dKt[T][4 * q4 + 1];
        k4.z += a.scale * dKt[T][4 * q4 + 2];
        k4.w += a.scale * dKt[T][4 * q4 + 3];
        v4.x += dVt[T][4 * q4 + 0];
        v4.y += dVt[T][4 * q4 + 1];
        v4.z += dVt[T][4 * q4 + 2];
        v4.w += dVt[T][4 * q4 + 3];
        *reinterpret_cast<float4*>(dkr + d0) = k4;
        *reinterpret_cast<float4*>(dvr + d0) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup = 4 waves x 32 queries of one query head.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq(const BwdArgs a) {
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int OFF_V = L::RBUF, OFF_KT = 2 * L::RBUF, BUF = 2 * L::RBUF + L::TBUF;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int item = xcd_item(a.n_items, a.per_xcd);
  if (item < 0) return;
  const int qt_rel = item % a.n_tiles;
  const int rest = item / a.n_tiles;
  const int hidx = rest % a.Hq, b = rest / a.Hq;
  const int h = a.head_order[hidx], g = a.kv_of[h];
  const int q0 = (a.n_tiles - 1 - qt_rel) * 128;  // latest (heaviest) query tiles first
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int qw0 = q0 + 32 * wv;
  const int qi = qw0 + n;
  const int qc = min(qi, a.Cq - 1);
  const float c = a.scale_log2;

  const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + b * a.q_bs + h * a.q_hs;
  const __bf16* db = reinterpret_cast<const __bf16*>(a.dout) + b * a.q_bs + h * a.q_hs;
  bf16x8 qreg[KS], dreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qreg[s] = *reinterpret_cast<const bf16x8*>(qb + (int64_t)qc * D + 16 * s + 8 * hh);
    dreg[s] = *reinterpret_cast<const bf16x8*>(db + (int64_t)qc * D + 16 * s + 8 * hh);
  }
  // rows past Cq read the padding: lse2 = +inf, so their probabilities are 0
  const float lse2 = a.lse2[b * a.l_bs + h * a.l_hs + qi];
  const float dlt = a.delta[b * a.l_bs + h * a.l_hs + qi];
  const int qpos = pos_of(a.qp, qc);
  const int wave_qmin = pos_of(a.qp, min(qw0, a.Cq - 1));
  const int wg_qmax = pos_of(a.qp, min(q0 + 127, a.Cq - 1));
  const int n_keys = a.causal ? allowed_prefix(a.kp, wg_qmax) : a.Ck;
  const int n_kt = (n_keys + 63) / 64;

  floatx16 dQt[DT];
#pragma unroll
  for (int T = 0; T < DT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) dQt[T][i] = 0.f;

  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + b * a.k_bs + g * a.k_hs;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + b * a.k_bs + g * a.k_hs;
  const __bf16* ktb = reinterpret_cast<const __bf16*>(a.kt) + b * a.kt_bs + g * a.kt_hs;
  auto load_tile = [&](int t, int buf) {
    const int kb0 = t * 64;
    unsigned char* B0 = lds + buf * BUF;
    load_row_tile<D>(kb + (int64_t)kb0 * D, a.Ck - 1 - kb0, B0, wv, lane);
    load_row_tile<D>(vb + (int64_t)kb0 * D, a.Ck - 1 - kb0, B0 + OFF_V, wv, lane);
    load_trans_tile<D>(ktb + kb0, a.Ckp, B0 + OFF_KT, wv, lane);
  };
  const int rbase = kperm(n) * L::ROW + hh * 16;
  if (n_kt > 0) load_tile(0, 0);
  for (int t = 0; t < n_kt; ++t) {
    lds_loads_barrier();
    if (t + 1 < n_kt) load_tile(t + 1, (t + 1) & 1);
    const unsigned char* B0 = lds + (t & 1) * BUF;
    const int kb0 = t * 64;
    const bool need_mask =
        kb0 + 64 > a.Ck || (a.causal && pos_of(a.kp, min(kb0 + 63, a.Ck - 1)) > wave_qmin);
    bf16x8 dSb[4];
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      // S^T, dP^T for 32 keys (kperm rows) x this wave's 32 queries; element i
      // of a lane is key 32th + 16(i/8) + 8hh + i%8 of the tile
      floatx16 S, dP;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        S[i] = 0.f;
        dP[i] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(B0 + rbase + th * 32 * L::ROW + s * 32);
        const bf16x8 va =
            *reinterpret_cast<const bf16x8*>(B0 + OFF_V + rbase + th * 32 * L::ROW + s * 32);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dreg[s], dP, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sc = S[i] * c - lse2;
        if (need_mask) {
          const int key = kb0 + 32 * th + 16 * (i >> 3) + 8 * hh + (i & 7);
          sc = masked(sc, key, a.Ck, a.causal, a.kp, qpos);
        }
        const float p = __builtin_amdgcn_exp2f(sc);
        dSb[2 * th + (i >> 3)][i & 7] = (__bf16)(p * (dP[i] - dlt));
      }
    }
    // dQ^T += K^T dS^T (A: row d of the K^T tile, keys 16u + 8h ..)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int T = 0; T < DT; ++T) {
        const bf16x8 kta = *reinterpret_cast<const bf16x8*>(
            B0 + OFF_KT + (32 * T + n) * L::TROW + (16 * u + 8 * hh) * 2);
        dQt[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kta, dSb[u], dQt[T], 0, 0, 0);
      }
  }

  if (qi < a.Cq) {
    float* dqr = a.dq + b * a.dq_bs + h * a.dq_hs + (int64_t)qi * D;
#pragma unroll
    for (int T = 0; T < DT; ++T)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * T + 8 * q4 + 4 * hh;
        float4 x = *reinterpret_cast<float4*>(dqr + d0);
        x.x += a.scale * dQt[T][4 * q4 + 0];
        x.y += a.scale * dQt[T][4 * q4 + 1];
        x.z += a.scale * dQt[T][4 * q4 + 2];
        x.w += a.scale * dQt[T][4 * q4 + 3];
        *reinterpret_cast<float4*>(dqr + d0) = x;
      }
  }
}

// ---------------------------------------------------------------------------
// delta = <dout, out> and lse in exp2 units, per query row, padded.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* __restrict__ out,
                                                       const __bf16* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ lse2p,
                                                       float* __restrict__ deltap,
                                                       int64_t rows_total, int64_t nblk,
                                                       int64_t C, int64_t Cp, int64_t o_bh,
                                                       int64_t l_bh) {
  constexpr int LPR = D / 8;     // lanes per row, 8 elements each
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int sub = lane / LPR, e = lane % LPR;
  for (int64_t r0 = ((int64_t)blockIdx.x * 4 + wv) * RPW; r0 < rows_total;
       r0 += (int64_t)gridDim.x * 4 * RPW) {
    const int64_t row = r0 + sub;
    const bool inr = row < rows_total;
    int64_t bh = 0, blk = 0, i = 0;
    if (inr) {
      bh = row / (nblk * Cp);
      const int64_t rr = row - bh * nblk * Cp;
      blk = rr / Cp;
      i = rr - blk * Cp;
    }
    const bool valid = inr && i < C;
    float acc = 0.f;
    if (valid) {
      const int64_t src = bh * o_bh + (blk * C + i) * D + e * 8;
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(out + src);
      const bf16x8 d = *reinterpret_cast<const bf16x8*>(dout + src);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fmaf((float)o[j], (float)d[j], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (inr && e == 0) {
      float l2 = INFINITY;
      if (valid) {
        const float l = lse[bh * l_bh + blk * C + i];
        l2 = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
      }
      deltap[row] = valid ? acc : 0.f;
      lse2p[row] = l2;
    }
  }
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float4* __restrict__ src,
                                                          __bf16* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4 x = src[i];
    bf16x4 y;
    y[0] = (__bf16)x.x;
    y[1] = (__bf16)x.y;
    y[2] = (__bf16)x.z;
    y[3] = (__bf16)x.w;
    *reinterpret_cast<bf16x4*>(dst + 4 * i) = y;
  }
}

template <int D>
constexpr size_t dkdv_lds_bytes() {
  return (size_t)2 * (2 * BwdLds<D>::RBUF + 2 * BwdLds<D>::TBUF + 512);
}
template <int D>
constexpr size_t dq_lds_bytes() {
  return (size_t)2 * (2 * BwdLds<D>::RBUF + BwdLds<D>::TBUF);
}

template <typename K>
hipError_t launch_big(K kern, size_t lds, int grid, const BwdArgs& a, hipStream_t s) {
  static_assert(sizeof(BwdArgs) <= 4096, "kernel arguments");
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a, int D, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  const int grid = a.per_xcd * kXcds;
  if (D == 128) return launch_big(attn_bwd_dkdv<128>, dkdv_lds_bytes<128>(), grid, a, s);
  return launch_big(attn_bwd_dkdv<64>, dkdv_lds_bytes<64>(), grid, a, s);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int D, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  const int grid = a.per_xcd * kXcds;
  if (D == 128) return launch_big(attn_bwd_dq<128>, dq_lds_bytes<128>(), grid, a, s);
  return launch_big(attn_bwd_dq<64>, dq_lds_bytes<64>(), grid, a, s);
}

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* lse2p,
                           float* deltap, int64_t BH, int64_t nblk, int64_t C, int64_t Cp, int D,
                           int64_t o_bh, int64_t l_bh, hipStream_t s) {
  const int64_t rows = BH * nblk * Cp;
  if (rows == 0) return hipSuccess;
  const int rows_per_block = 4 * (64 / (D / 8));
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  const __bf16* o = reinterpret_cast<const __bf16*>(out);
  const __bf16* d = reinterpret_cast<const __bf16*>(dout);
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, grid, dim3(256), 0, s, o, d, lse, lse2p, deltap, rows,
                       nblk, C, Cp, o_bh, l_bh);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, grid, dim3(256), 0, s, o, d, lse, lse2p, deltap, rows,
                       nblk, C, Cp, o_bh, l_bh);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                     dim3(256), 0, s, reinterpret_cast<const float4*>(src),
                     reinterpret_cast<__bf16*>(dst), n4);
  return hipGetLastError();
}

}  // namespace ra
