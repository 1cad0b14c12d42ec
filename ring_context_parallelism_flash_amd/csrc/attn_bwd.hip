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
//  * attn_bwd_dq: a workgroup owns 256 queries of one query head, two waves
//    per SIMD (Q and dO rows of a wave in registers, as in the forward) and
//    walks the key tiles (64 keys): S^T = K Q^T and dP^T = V dO^T with
//    kperm'd key rows, then dQ^T += K^T dS^T with a K^T tile in LDS.
//  * All tiles move global->LDS with direct 16-byte loads into padded rows
//    (bank-conflict-free operand reads), double buffered. Both kernels add into fp32 accumulators, so the ring can sum the
//    contributions of all block pairs.
#include <string.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "attn_common.h"
#include "attn_bwd_dkdv_loop.h"
#include "attn_bwd_dq_w64_loop.h"

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
template <int D, int NW = 4>
__device__ __forceinline__ void load_row_tile(const __bf16* base, int rows_left, unsigned char* dst,
                                              int wv, int lane) {
  using L = BwdLds<D>;
#pragma unroll
  for (int j = 0; j < (L::RINS + NW - 1) / NW; ++j) {
    const int ins = wv + NW * j;
    if (ins < L::RINS) {
      const int P = ins * 64 + lane;
      const int cch = P % L::RCPR;
      const int row = min(P / L::RCPR, rows_left);
      load_lds16(base + (int64_t)row * D + (cch < L::CPR ? cch : 0) * 8, dst + ins * 1024);
    }
  }
}

// Columns [0, 64) of a transposed [D][ld] array into padded LDS rows.
template <int D, int NW = 4>
__device__ __forceinline__ void load_trans_tile(const __bf16* base, int64_t ld, unsigned char* dst,
                                                int wv, int lane) {
  using L = BwdLds<D>;
#pragma unroll
  for (int j = 0; j < (L::TINS + NW - 1) / NW; ++j) {
    const int ins = wv + NW * j;
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

// 16-byte LDS read of four floats, issued by inline asm like the operand
// rings: the compiler waits for every outstanding direct global->LDS load
// before an LDS read it issues itself (it cannot tell that the read does not
// alias the loads' destination), which would drain the tile prefetch.
// The hardware writes the result register when the read returns; callers
// wait with an s_waitcnt that names the register as an operand.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int OFF>
__device__ __forceinline__ f32x4 ds_read_f4(unsigned addr) {
  f32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// First row of a block whose position is >= P (rows if none); positions
// increase with the row index.
__device__ __forceinline__ int first_row_at(const PosDesc& p, int rows, int P) {
  const int seg0 = p.nseg == 2 ? p.seg : rows;
  const int last0 = p.start0 + (seg0 - 1) * p.stride;
  if (P <= last0) return P <= p.start0 ? 0 : (P - p.start0 + p.stride - 1) / p.stride;
  if (p.nseg == 2 && P <= p.start1 + (p.seg - 1) * p.stride)
    return p.seg + (P <= p.start1 ? 0 : (P - p.start1 + p.stride - 1) / p.stride);
  return rows;
}

// dV^T += dO^T P and dK^T += Q^T dS for one 32-query sub-tile: 4*DT MFMAs
// whose A operands (rows d of the dO^T / Q^T tiles) stream from LDS through a
// ring of PF registers with an explicit wait before each use. Operand i:
// u = i / (2 DT) (16-query half), T = (i / 2) % DT (32-wide d tile), even i
// feed dV from dO^T, odd i feed dK from Q^T.
template <int D, int TROW, int TBUF>
struct DkdvStream {
  static constexpr int DT = D / 32, N = 4 * DT, PF = 4;
  static_assert(N >= PF, "fewer operands than reads in flight");
  static constexpr int off(int i) {
    return ((i & 1) ? 0 : TBUF) + 32 * ((i >> 1) % DT) * TROW + 32 * (i / (2 * DT));
  }
  template <int I>
  static __device__ __forceinline__ void step(unsigned ta, bf16x8 (&r)[PF], floatx16 (&dVt)[DT],
                                              floatx16 (&dKt)[DT], const bf16x8 (&Pb)[2],
                                              const bf16x8 (&dSb)[2]) {
    lds_wait<(N - 1 - I < PF - 1) ? (N - 1 - I) : (PF - 1)>(r[I % PF]);
    constexpr int T = (I >> 1) % DT, u = I / (2 * DT);
    if constexpr ((I & 1) == 0)
      dVt[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], Pb[u], dVt[T], 0, 0, 0);
    else
      dKt[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], dSb[u], dKt[T], 0, 0, 0);
    if constexpr (I + PF < N) r[I % PF] = ds_read16<off(I + PF)>(ta);
    if constexpr (I + 1 < N) step<I + 1>(ta, r, dVt, dKt, Pb, dSb);
  }
  template <int I>
  static __device__ __forceinline__ void prefetch(unsigned ta, bf16x8 (&r)[PF]) {
    r[I] = ds_read16<off(I)>(ta);
    if constexpr (I + 1 < PF) prefetch<I + 1>(ta, r);
  }
  static __device__ __forceinline__ void run(unsigned ta, floatx16 (&dVt)[DT], floatx16 (&dKt)[DT],
                                             const bf16x8 (&Pb)[2], const bf16x8 (&dSb)[2]) {
    bf16x8 r[PF];
    prefetch<0>(ta, r);
    step<0>(ta, r, dVt, dKt, Pb, dSb);
  }
};

// S = Q K^T and dP = dO V^T for one 32-query sub-tile: 2*KS MFMAs whose A
// operands (kperm'd Q / dO rows) stream from LDS through a ring of PF
// registers. Operand i: s = i / 2 (16-wide d step), even i = Q (S), odd i =
// dO (dP). After MFMA i the functor `work` gets step i, so a caller can
// spread independent arithmetic over the matrix work.
template <int D, int ROW, int RBUF>
struct SdpStream {
  static constexpr int KS = D / 16, N = 2 * KS, PF = 4;
  static constexpr int off(int i) { return ((i & 1) ? RBUF : 0) + 32 * (i >> 1); }
  template <int I, class W>
  static __device__ __forceinline__ void step(unsigned ra, bf16x8 (&r)[PF], const bf16x8 (&kreg)[KS],
                                              const bf16x8 (&vreg)[KS], floatx16& S, floatx16& dP,
                                              W& work) {
    lds_wait<(N - 1 - I < PF - 1) ? (N - 1 - I) : (PF - 1)>(r[I % PF]);
    if constexpr ((I & 1) == 0)
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], kreg[I >> 1], S, 0, 0, 0);
    else
      dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], vreg[I >> 1], dP, 0, 0, 0);
    if constexpr (I + PF < N) r[I % PF] = ds_read16<off(I + PF)>(ra);
    work(std::integral_constant<int, I>{});
    if constexpr (I + 1 < N) step<I + 1>(ra, r, kreg, vreg, S, dP, work);
  }
  template <int I>
  static __device__ __forceinline__ void prefetch(unsigned ra, bf16x8 (&r)[PF]) {
    r[I] = ds_read16<off(I)>(ra);
    if constexpr (I + 1 < PF) prefetch<I + 1>(ra, r);
  }
  template <class W>
  static __device__ __forceinline__ void run(unsigned ra, const bf16x8 (&kreg)[KS],
                                             const bf16x8 (&vreg)[KS], floatx16& S, floatx16& dP,
                                             W& work) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] = 0.f;
      dP[i] = 0.f;
    }
    bf16x8 r[PF];
    prefetch<0>(ra, r);
    step<0>(ra, r, kreg, vreg, S, dP, work);
  }
};

// The S, dP stream of the next sub-tile followed by the dV, dK stream of
// this one, as ONE operand stream: N1 = 2*KS reads from the Q / dO rows (ra)
// then N2 = 4*DT from the Q^T / dO^T tiles (ta), PF in flight through one
// register ring with counted waits over the whole sequence. The last PF
// steps of the first part issue the first reads of the second, so the dV /
// dK MFMAs start without an LDS round trip of their own. `work` runs after
// each of the first N1 MFMAs (it must finish P, dS by then).
template <class G1, class G2>
struct SdpDkdvStream {
  static constexpr int N1 = G1::N, N2 = G2::N, N = N1 + N2, PF = 4;
  static constexpr int KS = G1::KS, DT = G2::DT;
  template <int I>
  static __device__ __forceinline__ bf16x8 read(unsigned ra, unsigned ta) {
    if constexpr (I < N1)
      return ds_read16<G1::off(I)>(ra);
    else
      return ds_read16<G2::off(I - N1)>(ta);
  }
  template <int I, class W>
  static __device__ __forceinline__ void step(unsigned ra, unsigned ta, bf16x8 (&r)[PF],
                                              const bf16x8 (&kreg)[KS], const bf16x8 (&vreg)[KS],
                                              floatx16& S, floatx16& dP, floatx16 (&dVt)[DT],
                                              floatx16 (&dKt)[DT], const bf16x8 (&Pb)[2],
                                              const bf16x8 (&dSb)[2], W& work) {
    lds_wait<(N - 1 - I < PF - 1) ? (N - 1 - I) : (PF - 1)>(r[I % PF]);
    if constexpr (I < N1) {
      if constexpr ((I & 1) == 0)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], kreg[I >> 1], S, 0, 0, 0);
      else
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], vreg[I >> 1], dP, 0, 0, 0);
    } else {
      constexpr int i = I - N1, T = (i >> 1) % DT, u = i / (2 * DT);
      if constexpr ((i & 1) == 0)
        dVt[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], Pb[u], dVt[T], 0, 0, 0);
      else
        dKt[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], dSb[u], dKt[T], 0, 0, 0);
    }
    if constexpr (I + PF < N) r[I % PF] = read<I + PF>(ra, ta);
    if constexpr (I < N1) work(std::integral_constant<int, I>{});
    if constexpr (I + 1 < N) step<I + 1>(ra, ta, r, kreg, vreg, S, dP, dVt, dKt, Pb, dSb, work);
  }
  template <int I>
  static __device__ __forceinline__ void prefetch(unsigned ra, unsigned ta, bf16x8 (&r)[PF]) {
    r[I] = read<I>(ra, ta);
    if constexpr (I + 1 < PF) prefetch<I + 1>(ra, ta, r);
  }
  template <class W>
  static __device__ __forceinline__ void run(unsigned ra, unsigned ta, const bf16x8 (&kreg)[KS],
                                             const bf16x8 (&vreg)[KS], floatx16& S, floatx16& dP,
                                             floatx16 (&dVt)[DT], floatx16 (&dKt)[DT],
                                             const bf16x8 (&Pb)[2], const bf16x8 (&dSb)[2],
                                             W& work) {
    static_assert(N1 >= PF && N2 >= PF, "fewer operands than reads in flight");
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] = 0.f;
      dP[i] = 0.f;
    }
    bf16x8 r[PF];
    prefetch<0>(ra, ta, r);
    step<0>(ra, ta, r, kreg, vreg, S, dP, dVt, dKt, Pb, dSb, work);
  }
};

// P = exp2(S c - lse2) and dS = P (dP - delta) of a 32-query sub-tile,
// rounded to bf16 (the B operands of the dV / dK products), PER elements per
// step of the next sub-tile's S / dP stream. Element e = 8w + jj of a lane is
// row offset 16w + jj of the sub-tile; causal: masked iff that offset is
// below lim.
template <int PER, bool MASK>
struct DkdvProbs {
  const floatx16& S;
  const floatx16& dP;
  f32x4 (&lx)[4];  // lse2 of rows 16w + jj: lx[2w + jj/4][jj%4]
  f32x4 (&dx)[4];  // minus delta, same layout
  float c;
  int lim;
  bf16x8 (&Pb)[2];
  bf16x8 (&dSb)[2];
  template <int I>
  __device__ __forceinline__ void operator()(std::integral_constant<int, I>) {
    if constexpr (I == 0) {
      // lx / dx are LDS reads issued before the stream; its first counted
      // wait (just executed) retired them, since LDS reads return in order.
      // Naming the registers here keeps every use below that wait.
      asm volatile("" : "+v"(lx[0]), "+v"(lx[1]), "+v"(lx[2]), "+v"(lx[3]), "+v"(dx[0]),
                   "+v"(dx[1]), "+v"(dx[2]), "+v"(dx[3]));
    }
#pragma unroll
    for (int e = I * PER; e < (I + 1) * PER; ++e) {
      const int w = e >> 3, jj = e & 7;
      const float l2 = lx[2 * w + (jj >> 2)][jj & 3];
      const float ndl = dx[2 * w + (jj >> 2)][jj & 3];
      float sc = fmaf(S[e], c, -l2);
      if constexpr (MASK) sc = (16 * w + jj < lim) ? -INFINITY : sc;
      const float p = __builtin_amdgcn_exp2f(sc);
      Pb[w][jj] = (__bf16)p;
      dSb[w][jj] = (__bf16)(p * (dP[e] + ndl));
    }
  }
};
struct NoWork {
  template <int I>
  __device__ __forceinline__ void operator()(std::integral_constant<int, I>) {}
};
// A stream's per-MFMA work followed by one tile load (loads(step) decides
// which, if any).
template <class W, class LD>
struct WithLoads {
  W& work;
  LD& loads;
  template <int I>
  __device__ __forceinline__ void operator()(std::integral_constant<int, I> i) {
    work(i);
    loads(i);
  }
};

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 4 waves x 32 keys of one KV head, one wave per SIMD.
//
// The 64-query tiles of every query head that reads the KV head form one
// stream (tile-major, latest tile first), walked in 32-query sub-tiles j = 0,
// 1, ... Iteration j issues the
// S and dP MFMAs of sub-tile j+1 with the probability arithmetic of sub-tile
// j spread between them (the VALU work runs under the wave's own matrix
// work), then the dV and dK MFMAs of sub-tile j. The two MFMA groups read
// their LDS operands through one explicit register ring (SdpDkdvStream), so
// the dV / dK operands are in flight before the S / dP MFMAs end, and the
// sub-tile's lse2 / delta reads are retired by that ring's first counted
// wait (an odd sub-tile's already before the barrier). LDS holds two buffers of
// Q / dO rows (read by the S, dP products) and two of Q^T / dO^T plus the
// rows' lse2 and delta (read by the dV, dK products and the arithmetic).
// Rows of tile u+2 are loaded at the start of iteration 2u+1 and Q^T/dO^T of
// tile u+2 at the start of iteration 2u+2: each load has two iterations to
// land before the barrier that publishes it.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv(const BwdArgs a) {
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int ROWS_BUF = 2 * L::RBUF;  // Q rows, dO rows
  // lse2 and delta get 1 KiB each: the wave that loads them uses all 64
  // lanes (lanes 16..63 repeat lanes 0..15), so every counted load is a
  // whole-wave instruction
  constexpr int OFF_L = 2 * L::TBUF, OFF_DL = OFF_L + 1024;
  constexpr int TRANS_BUF = 2 * L::TBUF + 2048;  // Q^T, dO^T, lse2, delta
  constexpr int OFF_TRANS = 2 * ROWS_BUF;
  constexpr int OFF_HTAB = OFF_TRANS + 2 * TRANS_BUF;  // kMaxHeads ints
  using G1 = SdpStream<D, L::ROW, L::RBUF>;
  using G2 = DkdvStream<D, L::TROW, L::TBUF>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int item = xcd_item(a.n_items, a.per_xcd);
  if (item < 0) return;
  const int kt = item % a.n_tiles;
  const int rest = item / a.n_tiles;
  const int g = rest % a.Hkv, b = rest / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: load branches are per wave
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
    // K and V are only ever MFMA operands: keep them in AGPRs, which leaves
    // the VGPRs to the probability arithmetic
    asm volatile("" : "+a"(kreg[s]));
    asm volatile("" : "+a"(vreg[s]));
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
  // causal: this lane's key is seen by query rows >= row_min only
  const int row_min = a.causal ? first_row_at(a.qp, a.Cq, kpos) : 0;
  const int wg_kmin = pos_of(a.kp, min(k0, a.Ck - 1));
  // query rows before the first one that sees a key of this workgroup
  const int q_lo = a.causal ? allowed_prefix(a.qp, wg_kmin - 1) : 0;
  const int t_lo = q_lo / 64;
  const int n_t = max(0, (a.Cq + 63) / 64 - t_lo);
  const int g0 = a.grp_off[g], ng = a.grp_off[g + 1] - g0;
  const int NT = ng * n_t;  // tiles in the stream
  // The group's query heads go to an LDS table once: a runtime-indexed read
  // of the kernel-argument array inside the loop would be a vector-memory
  // load, and waiting for it would also drain the in-flight tile loads.
  int* htab = reinterpret_cast<int*>(lds + OFF_HTAB);
  if (tid < ng) htab[tid] = a.head_order[g0 + tid];
  // Up to 64 heads also sit one per lane of a register (loaded with the
  // table, published by the same barrier): v_readlane returns head i with no
  // memory access, where the table read leaves this wave -- the only one on
  // its SIMD -- waiting for an LDS round trip.
  const bool heads_in_lanes = ng <= 64;
  const int vhead = (lane < ng) ? (int)a.head_order[g0 + lane] : 0;
  auto head_at = [&](int i) -> int {  // i wave-uniform; the table is published
    if (heads_in_lanes) return __builtin_amdgcn_readlane(vhead, i);
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v)
                 : "v"(lds_addr(htab + i))
                 : "memory");
    return __builtin_amdgcn_readfirstlane(v);
  };
  const int NJ = 2 * NT;                         // sub-tiles (even)
  const int rbase = kperm(n) * L::ROW + hh * 16;  // A operand of S / dP (+32 rows per sub-tile)
  // Direct loads per batch: the 1 KiB loads of a tile are dealt round-robin
  // to the 4 waves, so a wave issues at least VM_MIN of them in either batch
  // (rows: 2 tiles of RINS; transposed: 2 of TINS, plus lse2 / delta on
  // waves 0 / 1). Loads complete in order, so waiting until at most VM_MIN
  // are outstanding retires every older batch.
  constexpr int VM_MIN = 2 * ((L::RINS < L::TINS ? L::RINS : L::TINS) / 4);

  struct TileSrc {
    int h, q0;
  };
  // Stream order: query tiles from the last down to t_lo, and for each tile
  // every query head of the group. All workgroups of a KV head start on the
  // block's last tile and move down together (where t_lo differs -- a causal
  // diagonal block -- the shorter ranges just end earlier), so they read the
  // same Q / dO tiles at about the same time and share them in L2.
  auto tile_src = [&](int T) -> TileSrc {
    const int tr = T / ng;
    return TileSrc{head_at(T - tr * ng), (t_lo + n_t - 1 - tr) * 64};
  };
  auto load_rows = [&](int T) {
    const TileSrc ts = tile_src(T);
    const int64_t off = b * a.q_bs + ts.h * a.q_hs + (int64_t)ts.q0 * D;
    unsigned char* B0 = lds + (T & 1) * ROWS_BUF;
    load_row_tile<D>(reinterpret_cast<const __bf16*>(a.q) + off, a.Cq - 1 - ts.q0, B0, wv, lane);
    load_row_tile<D>(reinterpret_cast<const __bf16*>(a.dout) + off, a.Cq - 1 - ts.q0,
                     B0 + L::RBUF, wv, lane);
  };
  auto load_trans = [&](int T) {
    const TileSrc ts = tile_src(T);
    const int64_t toff = b * a.qt_bs + ts.h * a.qt_hs + ts.q0;
    const int64_t loff = b * a.l_bs + ts.h * a.l_hs + ts.q0;
    unsigned char* B0 = lds + OFF_TRANS + (T & 1) * TRANS_BUF;
    load_trans_tile<D>(reinterpret_cast<const __bf16*>(a.qt) + toff, a.Cqp, B0, wv, lane);
    load_trans_tile<D>(reinterpret_cast<const __bf16*>(a.dot) + toff, a.Cqp, B0 + L::TBUF, wv,
                       lane);
    if (wv == 0) load_lds16(a.lse2 + loff + 4 * (lane & 15), B0 + OFF_L);
    if (wv == 1) load_lds16(a.ndelta + loff + 4 * (lane & 15), B0 + OFF_DL);
  };
  // LDS address of the A operands of S / dP for sub-tile jn: kperm'd rows, so
  // element i of a lane's result is query 32(jn%2) + 16(i/8) + 8hh + i%8
  auto g1_addr = [&](int jn) -> unsigned {
    return lds_addr(lds + ((jn >> 1) & 1) * ROWS_BUF) + rbase + (jn & 1) * 32 * L::ROW;
  };

  // Per-lane parts of this wave's direct loads (chunk ins = wv + 4j of a
  // tile): row and byte offset within a 64-row tile, byte offset within a
  // transposed tile. The loads of an iteration go out one per MFMA of its
  // S / dP stream rather than in a burst after the barrier, where they would
  // stall all four waves at once.
  constexpr int LJ = (L::TINS + 3) / 4;  // most chunk loads of one tile per wave
  static_assert(L::RINS <= L::TINS, "row tiles take no more loads than transposed ones");
  uint32_t rrow[LJ], rch[LJ], tofs[LJ];
#pragma unroll
  for (int jj = 0; jj < LJ; ++jj) {
    const int P = (wv + 4 * jj) * 64 + lane;
    const int cr = P % L::RCPR, ct = P % 9;
    rrow[jj] = (uint32_t)(P / L::RCPR);
    rch[jj] = (uint32_t)(cr < L::CPR ? cr : 0) * 16u;
    tofs[jj] = ((uint32_t)(P / 9) * (uint32_t)a.Cqp + (uint32_t)(ct < 8 ? ct : 0) * 8u) * 2u;
  }
  // lse2 / delta of sub-tile j (8 LDS reads into lx, dx). Sub-tiles 2m and
  // 2m+1 read the same Q^T / dO^T tile, published by the barrier of
  // iteration 2m and not overwritten before iteration 2m+2: the reads of the
  // odd sub-tile go out at the end of the even iteration and land across the
  // barrier; they are older than the operand stream's first reads, so its
  // first counted wait retires them.
  auto lse_reads = [&](int j, f32x4 (&lx)[4], f32x4 (&dx)[4]) {
    const unsigned char* TB = lds + OFF_TRANS + ((j >> 1) & 1) * TRANS_BUF;
    const unsigned la = lds_addr(TB) + (32 * (j & 1) + 8 * hh) * 4;
    lx[0] = ds_read_f4<OFF_L>(la);
    lx[1] = ds_read_f4<OFF_L + 16>(la);
    lx[2] = ds_read_f4<OFF_L + 64>(la);
    lx[3] = ds_read_f4<OFF_L + 80>(la);
    dx[0] = ds_read_f4<OFF_DL>(la);
    dx[1] = ds_read_f4<OFF_DL + 16>(la);
    dx[2] = ds_read_f4<OFF_DL + 64>(la);
    dx[3] = ds_read_f4<OFF_DL + 80>(la);
  };
  f32x4 lx[4], dx[4];
  auto iter = [&](auto mask, auto odd, int j, const floatx16& Sc, const floatx16& dPc,
                  floatx16& Sn, floatx16& dPn) {
    constexpr bool ODD = decltype(odd)::value;
    if (j > 0) {
      // the batch of two iterations ago has landed in this wave ...
      vm_wait<VM_MIN>();
      // ... and in every wave; every wave is done with iteration j-1 (its LDS
      // reads were all waited for)
      workgroup_barrier();
    }
    // This iteration's loads: an odd one the Q / dO rows of stream tile
    // (j >> 1) + 2, an even one the Q^T / dO^T tile (j >> 1) + 1 with its
    // lse2 / delta, each into the buffer that tile will use; a tile past the
    // stream's end repeats the last one (into a buffer nobody reads before it
    // is loaded again), so every iteration issues the same loads.
    const int Tu = ODD ? (j >> 1) + 2 : (j >> 1) + 1;
    const TileSrc ls = tile_src(min(Tu, NT - 1));
    const int rows_left = a.Cq - 1 - ls.q0;
    const unsigned char* src0;
    const unsigned char* src1;
    const float* src2;
    unsigned char* dst;
    if constexpr (ODD) {
      const int64_t off = b * a.q_bs + ls.h * a.q_hs + (int64_t)ls.q0 * D;
      src0 = reinterpret_cast<const unsigned char*>(reinterpret_cast<const __bf16*>(a.q) + off);
      src1 = reinterpret_cast<const unsigned char*>(reinterpret_cast<const __bf16*>(a.dout) + off);
      src2 = nullptr;
      dst = lds + (Tu & 1) * ROWS_BUF;
    } else {
      const int64_t toff = b * a.qt_bs + ls.h * a.qt_hs + ls.q0;
      src0 = reinterpret_cast<const unsigned char*>(reinterpret_cast<const __bf16*>(a.qt) + toff);
      src1 = reinterpret_cast<const unsigned char*>(reinterpret_cast<const __bf16*>(a.dot) + toff);
      src2 = (wv == 0 ? a.lse2 : a.ndelta) + b * a.l_bs + ls.h * a.l_hs + ls.q0 + 4 * (lane & 15);
      dst = lds + OFF_TRANS + (Tu & 1) * TRANS_BUF;
    }
    // step I < J: chunk I of the first tensor, J <= I < 2J: chunk I - J of
    // the second, I = 2J: lse2 (wave 0) or delta (wave 1)
    auto loads = [&](auto ic) {
      constexpr int I = decltype(ic)::value;
      static_assert(2 * LJ < G1::N, "every load has a step");
      if constexpr (I < 2 * LJ) {
        constexpr int jj = I % LJ;
        const int ins = wv + 4 * jj;
        if constexpr (ODD) {
          if (ins < L::RINS)
            load_lds16((I < LJ ? src0 : src1) + (min(rrow[jj], (uint32_t)rows_left) * (D * 2) + rch[jj]),
                       dst + (I < LJ ? 0 : L::RBUF) + ins * 1024);
        } else {
          if (ins < L::TINS)
            load_lds16((I < LJ ? src0 : src1) + tofs[jj], dst + (I < LJ ? 0 : L::TBUF) + ins * 1024);
        }
      } else if constexpr (I == 2 * LJ && !ODD) {
        if (wv < 2) load_lds16(src2, dst + (wv == 0 ? OFF_L : OFF_DL));
      }
    };
    const unsigned char* TB = lds + OFF_TRANS + ((j >> 1) & 1) * TRANS_BUF;
    const int r0 = 32 * (j & 1) + 8 * hh;  // rows r0 + 16w + jj of the tile
    // (tile_src reads the head table with a wait of its own: before the
    // uncounted lse2 / delta reads below)
    const int lim = row_min - (tile_src(j >> 1).q0 + r0);
    if (!(j & 1)) lse_reads(j, lx, dx);  // odd sub-tiles: issued by the even iteration
    bf16x8 Pb[2], dSb[2];
    DkdvProbs<16 / G1::N, decltype(mask)::value> pr{Sc, dPc, lx, dx, c, lim, Pb, dSb};
    WithLoads<decltype(pr), decltype(loads)> work{pr, loads};
    // the S, dP MFMAs of sub-tile j+1 (past the end: a stale but valid
    // buffer, result unused) with this sub-tile's arithmetic and the tile
    // loads between them, then this sub-tile's dV, dK MFMAs, in one operand
    // stream
    SdpDkdvStream<G1, G2>::run(g1_addr(min(j + 1, NJ - 1)), lds_addr(TB) + n * L::TROW + r0 * 2,
                               kreg, vreg, Sn, dPn, dVt, dKt, Pb, dSb, work);
    if (!(j & 1)) lse_reads(j + 1, lx, dx);  // NJ is even: an odd sub-tile follows
  };

  __syncthreads();  // the head table
  if (NT > 0) {
    load_rows(0);
    load_trans(0);
    if (NT > 1) {
      load_rows(1);
      load_trans(1);
    }
    lds_loads_barrier();
    floatx16 SA, dPA, SB, dPB;
    NoWork nw;
    G1::run(g1_addr(0), kreg, vreg, SA, dPA, nw);
    // Query tiles that start at or after every lane's first allowed row hold
    // no masked pair. The stream walks tiles latest first, so they are its
    // leading whole tiles (all heads of each): those sub-tiles run without
    // the mask's compare and select, the rest with them.
    // row_min grows with the key index (positions increase along a block),
    // so the wave's largest is its last key's: a scalar, with no cross-lane
    // shuffle -- a shuffle is an LDS-pipe instruction, and one placed among
    // the operand reads would upset their counted lgkmcnt waits.
    const int rmax =
        a.causal ? first_row_at(a.qp, a.Cq, pos_of(a.kp, min(kw0 + 31, a.Ck - 1))) : 0;
    const int j_free = 2 * ng * min(n_t, max(0, t_lo + n_t - (rmax + 63) / 64));
    int j = 0;
    for (; j < j_free; j += 2) {  // NJ and j_free are even
      iter(std::false_type{}, std::false_type{}, j, SA, dPA, SB, dPB);
      iter(std::false_type{}, std::true_type{}, j + 1, SB, dPB, SA, dPA);
    }
    for (; j < NJ; j += 2) {
      iter(std::true_type{}, std::false_type{}, j, SA, dPA, SB, dPB);
      iter(std::true_type{}, std::true_type{}, j + 1, SB, dPB, SA, dPA);
    }
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
// dK, dV for D = 128, one wave per SIMD: the workgroup and its query-tile
// stream are those of attn_bwd_dkdv, the loop over the stream -- the S / dP
// MFMAs of the next 32-query sub-tile with this one's P / dS arithmetic
// between them, then this sub-tile's dV / dK MFMAs, the causal mask and the
// tile loads -- is one inline-asm statement with a fixed schedule and fixed
// registers (attn_bwd_dkdv_loop.h, written by gen_bwd_dkdv_w32.py). The
// rows buffers also hold the tile's lse2 / delta, so a sub-tile's are read
// during the phase before its arithmetic.
// ---------------------------------------------------------------------------
constexpr size_t dkdv_w32_lds_bytes() {
  return 2 * (size_t)dkdvw::kRowsBuf + 2 * (size_t)dkdvw::kTransBuf;
}

template <bool RAGGED>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_w32(const BwdArgs a) {
  constexpr int D = 128, NW = 4, NC = dkdvw::kChunks;
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DT = D / 32;
  static_assert(dkdvw::kOffL == L::RBUF && dkdvw::kOffDO == L::RBUF + 1024 &&
                    dkdvw::kRowsBuf == 2 * L::RBUF + 2048 && dkdvw::kTransBuf == 2 * L::TBUF &&
                    L::RINS == 17 && L::TINS == 18 && NC * NW * 1024 == dkdvw::kRowsBuf &&
                    dkdv_w32_lds_bytes() <= 160 * 1024,
                "LDS layout of the one-wave-per-SIMD dK / dV kernel");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* Rows = lds;                         // [2][Q | lse2 | dO | minus delta]
  unsigned char* Trans = lds + 2 * dkdvw::kRowsBuf;  // [2][Q^T | dO^T]

  const int item = xcd_item(a.n_items, a.per_xcd);
  if (item < 0) return;
  const int kt = item % a.n_tiles;
  const int rest = item / a.n_tiles;
  const int g = rest % a.Hkv, b = rest / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int k0 = kt * 128, kw0 = k0 + 32 * wv;
  const int keyc = min(kw0 + n, a.Ck - 1);

  const int kpos = pos_of(a.kp, keyc);
  // causal: this lane's key is seen by query rows >= row_min only
  const int row_min = a.causal ? first_row_at(a.qp, a.Cq, kpos) : 0;
  const int wg_kmin = pos_of(a.kp, min(k0, a.Ck - 1));
  const int q_lo = a.causal ? allowed_prefix(a.qp, wg_kmin - 1) : 0;
  const int t_lo = q_lo / 64;
  const int n_t = max(0, (a.Cq + 63) / 64 - t_lo);
  const int g0 = a.grp_off[g], ng = a.grp_off[g + 1] - g0;
  const int NT = __builtin_amdgcn_readfirstlane(ng * n_t);  // tiles in the stream
  if (NT == 0) return;  // no query sees these keys: nothing to add

  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k) + b * a.k_bs + g * a.k_hs;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v) + b * a.k_bs + g * a.k_hs;
  bf16x8 kreg[KS], vreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kreg[s] = *reinterpret_cast<const bf16x8*>(kbase + (int64_t)keyc * D + 16 * s + 8 * hh);
    vreg[s] = *reinterpret_cast<const bf16x8*>(vbase + (int64_t)keyc * D + 16 * s + 8 * hh);
  }

  // The group's query heads, one per lane (ng <= 64): tile T of the stream
  // is head lane T % ng, queries from (t_lo + n_t - 1 - T / ng) * 64.
  const int vhead = (lane < ng) ? (int)a.head_order[g0 + lane] : 0;
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto head_at = [&](int i) { return uni(__builtin_amdgcn_readlane(vhead, i)); };
  auto q0_at = [&](int T) { return uni((t_lo + n_t - 1 - T / ng) * 64); };
  auto uni_ptr = [](const void* p) {
    const uint64_t v = (uint64_t)(size_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(size_t)(((uint64_t)hi << 32) | lo);
  };
  const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + b * a.q_bs;
  const __bf16* db = reinterpret_cast<const __bf16*>(a.dout) + b * a.q_bs;
  const __bf16* qtb = reinterpret_cast<const __bf16*>(a.qt) + b * a.qt_bs;
  const __bf16* dotb = reinterpret_cast<const __bf16*>(a.dot) + b * a.qt_bs;
  const float* lse2b = a.lse2 + b * a.l_bs;
  const float* ndlb = a.ndelta + b * a.l_bs;

  // prologue loads: rows (with lse2 / minus delta) of tiles 0 and 1 (the
  // last if the stream has one tile), the transposed tile 0
  auto load_rows = [&](int T, int buf) {
    const int h = head_at(T % ng), q0 = q0_at(T);
    unsigned char* B0 = Rows + buf * dkdvw::kRowsBuf;
    load_row_tile<D>(qb + h * a.q_hs + (int64_t)q0 * D, a.Cq - 1 - q0, B0, wv, lane);
    load_row_tile<D>(db + h * a.q_hs + (int64_t)q0 * D, a.Cq - 1 - q0, B0 + dkdvw::kOffDO, wv,
                     lane);
    if (wv == 1) load_lds16(lse2b + h * a.l_hs + q0 + 4 * (lane & 15), B0 + dkdvw::kOffL);
    if (wv == 3) load_lds16(ndlb + h * a.l_hs + q0 + 4 * (lane & 15), B0 + dkdvw::kOffDL);
  };
  load_rows(0, 0);
  load_rows(min(1, NT - 1), 1);
  {
    const int h = head_at(0), q0 = q0_at(0);
    load_trans_tile<D>(qtb + h * a.qt_hs + q0, a.Cqp, Trans, wv, lane);
    load_trans_tile<D>(dotb + h * a.qt_hs + q0, a.Cqp, Trans + L::TBUF, wv, lane);
  }

  // The loop's loads: wave w fills chunks 9w .. 9w+8 of each buffer. Rows:
  // waves 0 / 1 the Q rows (chunks 0-8 / 9-16) and w1 also lse2, waves 2 / 3
  // the dO rows and w3 also minus delta; transposed: waves 0 / 1 Q^T, 2 / 3
  // dO^T (chunks 0-8 / 9-17 of the tensor). Lane offsets of each load within
  // the tile, minus the load's own offset (loads 0-4 are placed from chunk
  // 4, loads 5-8 from chunk 8).
  unsigned rv[NC], rc[NC], tv[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const unsigned adj = (unsigned)((j < 5 ? 4 - j : 8 - j) * 1024);
    const int cj = NC * (wv & 1) + j;  // chunk within the tensor
    unsigned row, rch;
    if ((wv & 1) && j == NC - 1) {     // lse2 / minus delta: 64 floats, lanes 16+ repeat
      row = 0;
      rch = 16u * (lane & 15);
    } else {
      const int P = cj * 64 + lane, cr = P % L::RCPR;
      row = (unsigned)(P / L::RCPR);
      rch = (unsigned)(cr < L::CPR ? cr : 0) * 16u;
    }
    if (RAGGED) {
      rv[j] = row;
      rc[j] = rch + adj;
    } else {
      rv[j] = row * (D * 2) + rch + adj;
      rc[j] = 0;
    }
    const int P = cj * 64 + lane, ct = P % 9;
    tv[j] = ((unsigned)(P / 9) * (unsigned)a.Cqp + (unsigned)(ct < 8 ? ct : 0) * 8u) * 2u + adj;
  }
  // Query tiles that start at or after every lane's first allowed row hold
  // no masked pair; the stream walks tiles latest first, so they are its
  // leading sub-tiles. row_min grows with the key, so the wave's largest is
  // its last key's.
  const int rmax =
      a.causal ? first_row_at(a.qp, a.Cq, pos_of(a.kp, min(kw0 + 31, a.Ck - 1))) : 0;
  const int j_free = 2 * ng * min(n_t, max(0, t_lo + n_t - (rmax + 63) / 64));
  const unsigned lrows = lds_addr(Rows), ltrans = lds_addr(Trans);
  const void* lastb = wv == 0 ? (const void*)qb : wv == 1 ? (const void*)lse2b
                    : wv == 2 ? (const void*)db : (const void*)ndlb;
  lds_loads_barrier();

  floatx16 dVt[DT], dKt[DT];
  (RAGGED ? dkdvw::dkdv_loop_ragged : dkdvw::dkdv_loop)(
      NT, uni(j_free), uni(ng), head_at((NT - 1) % ng), q0_at(NT - 1), uni(a.Cq - 1),
      uni(lrows + (NC * wv + 4) * 1024), uni(ltrans + (NC * wv + 4) * 1024),
      uni((int)(a.q_hs * 2)), uni((int)(a.qt_hs * 2)),
      uni((wv & 1) ? (int)(a.l_hs * 4) : (int)(a.q_hs * 2)), uni((wv & 1) ? 2 : 8), a.scale_log2,
      uni_ptr(wv < 2 ? (const void*)qb : (const void*)db), uni_ptr(lastb),
      uni_ptr(wv < 2 ? (const void*)qtb : (const void*)dotb), lrows + kperm(n) * L::ROW + hh * 16,
      ltrans + n * L::TROW + hh * 16, lrows + 32 * hh, row_min - 8 * hh, vhead, rv, rc, tv, kreg,
      vreg, q0_at(0), q0_at(1), q0_at(2), head_at(1 % ng), head_at(2 % ng), uni(2 % ng), dVt,
      dKt);

  // epilogue: add into the fp32 accumulators; lane holds key kw0+n,
  // d = 32T + 8(i/4) + 4hh + i%4
  // (all 32 loads of the old values go out before the first store, which
  // the compiler cannot move them past: dk and dv might alias)
  const int key = kw0 + n;
  if (key < a.Ck) {
    float* dkr = a.dk + b * a.dk_bs + g * a.dk_hs + (int64_t)key * D;
    float* dvr = a.dv + b * a.dk_bs + g * a.dk_hs + (int64_t)key * D;
    float4 k4[DT * 4], v4[DT * 4];
#pragma unroll
    for (int j = 0; j < DT * 4; ++j) {
      const int d0 = 32 * (j >> 2) + 8 * (j & 3) + 4 * hh;
      k4[j] = *reinterpret_cast<const float4*>(dkr + d0);
      v4[j] = *reinterpret_cast<const float4*>(dvr + d0);
    }
#pragma unroll
    for (int T = 0; T < DT; ++T)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = 4 * T + q4, d0 = 32 * T + 8 * q4 + 4 * hh;
        k4[j].x += a.scale * dKt[T][4 * q4 + 0];
        k4[j].y += a.scale * dKt[T][4 * q4 + 1];
        k4[j].z += a.scale * dKt[T][4 * q4 + 2];
        k4[j].w += a.scale * dKt[T][4 * q4 + 3];
        v4[j].x += dVt[T][4 * q4 + 0];
        v4[j].y += dVt[T][4 * q4 + 1];
        v4[j].z += dVt[T][4 * q4 + 2];
        v4[j].w += dVt[T][4 * q4 + 3];
        *reinterpret_cast<float4*>(dkr + d0) = k4[j];
        *reinterpret_cast<float4*>(dvr + d0) = v4[j];
      }
  }
}

// dQ^T += K^T dS^T for one 32-key sub-tile: 2*DT MFMAs whose A operands
// (rows d of the K^T tile, 16 keys each) stream from LDS through a ring of PF
// registers. Operand i: u = i / DT (16-key half), T = i % DT (32-wide d tile).
template <int D, int TROW>
struct DqStream {
  static constexpr int DT = D / 32, N = 2 * DT, PF = 4;
  static_assert(N >= PF, "fewer operands than reads in flight");
  static constexpr int off(int i) { return 32 * (i % DT) * TROW + 32 * (i / DT); }
  template <int I>
  static __device__ __forceinline__ void step(unsigned ka, bf16x8 (&r)[PF], floatx16 (&dQt)[DT],
                                              const bf16x8 (&dSb)[2]) {
    lds_wait<(N - 1 - I < PF - 1) ? (N - 1 - I) : (PF - 1)>(r[I % PF]);
    dQt[I % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[I % PF], dSb[I / DT], dQt[I % DT], 0, 0, 0);
    if constexpr (I + PF < N) r[I % PF] = ds_read16<off(I + PF)>(ka);
    if constexpr (I + 1 < N) step<I + 1>(ka, r, dQt, dSb);
  }
  template <int I>
  static __device__ __forceinline__ void prefetch(unsigned ka, bf16x8 (&r)[PF]) {
    r[I] = ds_read16<off(I)>(ka);
    if constexpr (I + 1 < PF) prefetch<I + 1>(ka, r);
  }
  static __device__ __forceinline__ void run(unsigned ka, floatx16 (&dQt)[DT], const bf16x8 (&dSb)[2]) {
    bf16x8 r[PF];
    prefetch<0>(ka, r);
    step<0>(ka, r, dQt, dSb);
  }
};

// dS^T = P^T (dP^T - delta) of a 32-key sub-tile for the lane's query,
// rounded to bf16 (the B operands of the dQ product), PER elements per step of
// the next sub-tile's S^T / dP^T stream. Element e of a lane is key offset
// 16(e/8) + 8hh + e%8 of the sub-tile; it is masked iff 16(e/8) + e%8 >= lim
// (keys at or past the lane's allowed prefix, or past the block end).
template <int PER, bool MASK>
struct DqProbs {
  const floatx16& S;
  const floatx16& dP;
  float lse2, dlt, c;
  int lim;
  bf16x8 (&dSb)[2];
  template <int I>
  __device__ __forceinline__ void operator()(std::integral_constant<int, I>) {
#pragma unroll
    for (int e = I * PER; e < (I + 1) * PER; ++e) {
      float sc = fmaf(S[e], c, -lse2);
      if constexpr (MASK) sc = (16 * (e >> 3) + (e & 7) >= lim) ? -INFINITY : sc;
      const float p = __builtin_amdgcn_exp2f(sc);
      dSb[e >> 3][e & 7] = (__bf16)(p * (dP[e] - dlt));
    }
  }
};

// ---------------------------------------------------------------------------
// dQ: one workgroup = 8 waves x 32 queries of one query head, two waves per
// SIMD. The 64-key tiles are walked in 32-key sub-tiles j: iteration j issues
// the S^T and dP^T MFMAs of sub-tile j, the dS^T arithmetic, then the dQ
// MFMAs of sub-tile j, with no software pipelining inside a wave -- the
// SIMD's other wave fills the matrix pipe during one wave's arithmetic, and
// the registers a pipeline would hold (a second S^T / dP^T pair) are what
// lets two waves fit. K and V rows (read by S^T, dP^T) and K^T (read by dQ)
// have two LDS buffers each, shared by the 256 queries of the workgroup.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;  // waves per dq workgroup (32 queries each)

template <int D>
__global__ __launch_bounds__(64 * kDqWaves, 1) void attn_bwd_dq(const BwdArgs a) {
  constexpr int NW = kDqWaves;
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int ROWS_BUF = 2 * L::RBUF;  // K rows, V rows
  constexpr int TRANS_BUF = L::TBUF;     // K^T
  constexpr int OFF_TRANS = 2 * ROWS_BUF;
  using G1 = SdpStream<D, L::ROW, L::RBUF>;
  using G2 = DqStream<D, L::TROW>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int item = xcd_item(a.n_items, a.per_xcd);
  if (item < 0) return;
  const int qt_rel = item % a.n_tiles;
  const int rest = item / a.n_tiles;
  const int hidx = rest % a.Hq, b = rest / a.Hq;
  const int h = a.head_order[hidx], g = a.kv_of[h];
  const int q0 = (a.n_tiles - 1 - qt_rel) * (32 * NW);  // latest (heaviest) query tiles first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: load branches are per wave
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
    // only ever MFMA operands: keep them in AGPRs
    asm volatile("" : "+a"(qreg[s]));
    asm volatile("" : "+a"(dreg[s]));
  }
  // rows past Cq read the padding: lse2 = +inf, so their probabilities are 0
  // (rows past the padded length -- a 256-row workgroup can reach them --
  // read its last row; those rows' dq is never written)
  const int ql = min(qi, a.Cqp - 1);
  const float lse2 = a.lse2[b * a.l_bs + h * a.l_hs + ql];
  const float dlt = -a.ndelta[b * a.l_bs + h * a.l_hs + ql];
  const int qpos = pos_of(a.qp, qc);
  // keys this lane's query sees: a prefix of the block (positions increase)
  const int n_allow = a.causal ? allowed_prefix(a.kp, qpos) : a.Ck;
  const int wg_qmax = pos_of(a.qp, min(q0 + 32 * NW - 1, a.Cq - 1));
  const int n_keys = a.causal ? allowed_prefix(a.kp, wg_qmax) : a.Ck;
  const int NT = (n_keys + 63) / 64;  // key tiles
  const int NJ = 2 * NT;              // 32-key sub-tiles (even)

  floatx16 dQt[DT];
#pragma unroll
  for (int T = 0; T < DT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) dQt[T][i] = 0.f;

  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + b * a.k_bs + g * a.k_hs;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + b * a.k_bs + g * a.k_hs;
  const __bf16* ktb = reinterpret_cast<const __bf16*>(a.kt) + b * a.kt_bs + g * a.kt_hs;
  auto load_rows = [&](int T) {
    const int kb0 = T * 64;
    unsigned char* B0 = lds + (T & 1) * ROWS_BUF;
    load_row_tile<D, NW>(kb + (int64_t)kb0 * D, a.Ck - 1 - kb0, B0, wv, lane);
    load_row_tile<D, NW>(vb + (int64_t)kb0 * D, a.Ck - 1 - kb0, B0 + L::RBUF, wv, lane);
  };
  auto load_trans = [&](int T) {
    load_trans_tile<D, NW>(ktb + T * 64, a.Ckp, lds + OFF_TRANS + (T & 1) * TRANS_BUF, wv, lane);
  };
  const int rbase = kperm(n) * L::ROW + hh * 16;
  auto g1_addr = [&](int jn) -> unsigned {
    return lds_addr(lds + ((jn >> 1) & 1) * ROWS_BUF) + rbase + (jn & 1) * 32 * L::ROW;
  };
  // Tiles 0 and 1 are loaded up front; K, V rows and K^T of tile u+1 are
  // loaded at iteration 2u (u >= 1) into the buffers of tile u-1, which
  // every wave finished with in iteration 2u-1 (the barrier), and waited
  // for at iteration 2u+2, their first use (two iterations to land).
  if (NT > 0) {
    load_rows(0);
    load_trans(0);
    if (NT > 1) {
      load_rows(1);
      load_trans(1);
    }
    lds_loads_barrier();
    // Key tiles that end within every lane's allowed prefix hold no masked
    // pair (nor a key past the block end); they lead the walk and run
    // without the mask's compare and select. n_allow grows with the query
    // index, so the wave's smallest is its first query's: a scalar, with no
    // cross-lane shuffle (see the dK / dV kernel).
    const int amin = a.causal ? allowed_prefix(a.kp, pos_of(a.qp, min(qw0, a.Cq - 1))) : a.Ck;
    const int j_free = 2 * min(NT, max(0, amin) / 64);
    auto iter = [&](auto mask, int j) {
      if (j >= 2 && !(j & 1)) {
        vm_wait<0>();
        workgroup_barrier();
        if ((j >> 1) + 1 < NT) {
          load_rows((j >> 1) + 1);
          load_trans((j >> 1) + 1);
        }
      }
      floatx16 S, dP;
      NoWork nw;
      G1::run(g1_addr(j), qreg, dreg, S, dP, nw);
      bf16x8 dSb[2];
      const int lim = n_allow - ((j >> 1) * 64 + 32 * (j & 1) + 8 * hh);
      DqProbs<16, decltype(mask)::value> pr{S, dP, lse2, dlt, c, lim, dSb};
      pr(std::integral_constant<int, 0>{});
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      G2::run(lds_addr(lds + OFF_TRANS + ((j >> 1) & 1) * TRANS_BUF) + n * L::TROW +
                  (32 * (j & 1) + 8 * hh) * 2,
              dQt, dSb);
    };
    int j = 0;
    for (; j < j_free; ++j) iter(std::false_type{}, j);
    for (; j < NJ; ++j) iter(std::true_type{}, j);
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
// dQ for D = 128 blocks of whole 64-key tiles, one wave per SIMD: 4 waves x
// 64 query rows (two 32-row blocks per wave), so every K, V or K^T operand
// read from LDS feeds two MFMAs, one per row block. Q and dO stay in AGPRs;
// the key loop -- the S^T / dP^T MFMAs of the next 32-key sub-tile (dP^T
// accumulated from minus delta) with this one's dS arithmetic between them,
// then this sub-tile's dQ^T MFMAs, the
// causal mask and the tile loads -- is one inline-asm statement with a fixed
// schedule and fixed registers (attn_bwd_dq_w64_loop.h, written by
// gen_bwd_dq_w64.py). K and V row tiles rotate through three LDS buffers,
// K^T tiles through two; one barrier per 64-key tile.
// ---------------------------------------------------------------------------
constexpr int kDqW64Waves = 4;

constexpr size_t dq_w64_lds_bytes() {
  return (size_t)dqw64::kRowBufs * dqw64::kRowTileBytes + 2 * (size_t)dqw64::kKtBufBytes;
}

__global__ __launch_bounds__(64 * kDqW64Waves, 1) void attn_bwd_dq_w64(const BwdArgs a) {
  constexpr int D = 128, NW = kDqW64Waves;
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DT = D / 32;
  static_assert(dqw64::kRowTileBytes == 2 * L::RBUF && dqw64::kKtBufBytes == L::TBUF &&
                    L::RINS == 17 && L::TINS == 18 && dq_w64_lds_bytes() <= 160 * 1024,
                "LDS layout of the one-wave-per-SIMD dQ kernel");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* Rows = lds;                                           // [3][K 64 rows | V 64 rows]
  unsigned char* Kt = lds + dqw64::kRowBufs * dqw64::kRowTileBytes;  // [2][D][64 + 8]

  const int item = xcd_item(a.n_items, a.per_xcd);
  if (item < 0) return;
  const int qt_rel = item % a.n_tiles;
  const int rest = item / a.n_tiles;
  const int hidx = rest % a.Hq, b = rest / a.Hq;
  const int h = __builtin_amdgcn_readfirstlane((int)a.head_order[hidx]);
  const int g = __builtin_amdgcn_readfirstlane((int)a.kv_of[h]);
  const int q0 = (a.n_tiles - 1 - qt_rel) * (64 * NW);  // latest (heaviest) query tiles first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int qw0 = q0 + 64 * wv;
  const int qlast = a.Cq - 1;

  // the workgroup's keys: a prefix of the block (its last row sees the most)
  const int wg_qmax = pos_of(a.qp, min(q0 + 64 * NW - 1, qlast));
  const int n_keys = a.causal ? allowed_prefix(a.kp, wg_qmax) : a.Ck;
  const int n_kt = (n_keys + 63) / 64;
  if (n_kt == 0) return;  // nothing to add to dq

  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + b * a.k_bs + g * a.k_hs;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + b * a.k_bs + g * a.k_hs;
  const __bf16* ktb = reinterpret_cast<const __bf16*>(a.kt) + b * a.kt_bs + g * a.kt_hs;
  // The 1 KiB chunk loads of a tile are dealt round-robin to the waves, K
  // from wave 0, V from wave 1, K^T from wave 2, so each wave issues exactly
  // one fifth chunk load per tile (K: 17 chunks, V: 17, K^T: 18).
  const int wk = wv, wvv = (wv + 3) % NW, wt = (wv + 2) % NW;
  uint32_t koff[5], voff[5], toff[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int pk = (wk + NW * j) * 64 + lane, pv = (wvv + NW * j) * 64 + lane;
    const int pt = (wt + NW * j) * 64 + lane;
    const int ck = pk % L::RCPR, cv = pv % L::RCPR, ct = pt % 9;
    koff[j] = (uint32_t)((pk / L::RCPR) * D + (ck < L::CPR ? ck : 0) * 8) * 2u;
    voff[j] = (uint32_t)((pv / L::RCPR) * D + (cv < L::CPR ? cv : 0) * 8) * 2u;
    toff[j] = ((uint32_t)(pt / 9) * (uint32_t)a.Ckp + (uint32_t)(ct < 8 ? ct : 0) * 8u) * 2u;
  }
  // tile loads of the prologue (the loop issues the same ones)
  auto load_rows = [&](int t, int buf) {
    const unsigned char* ks = reinterpret_cast<const unsigned char*>(kb + (int64_t)t * 64 * D);
    const unsigned char* vs = reinterpret_cast<const unsigned char*>(vb + (int64_t)t * 64 * D);
    unsigned char* dst = Rows + buf * dqw64::kRowTileBytes;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      if (wk + NW * j < L::RINS) load_lds16(ks + koff[j], dst + (wk + NW * j) * 1024);
      if (wvv + NW * j < L::RINS) load_lds16(vs + voff[j], dst + L::RBUF + (wvv + NW * j) * 1024);
    }
  };
  auto load_kt = [&](int t, int buf) {
    const unsigned char* ts = reinterpret_cast<const unsigned char*>(ktb + t * 64);
    unsigned char* dst = Kt + buf * dqw64::kKtBufBytes;
#pragma unroll
    for (int j = 0; j < 5; ++j)
      if (wt + NW * j < L::TINS) load_lds16(ts + toff[j], dst + (wt + NW * j) * 1024);
  };
  load_rows(0, 0);
  if (n_kt > 1) load_rows(1, 1);
  load_kt(0, 0);

  // Q and dO of the wave's two blocks (rows past the block repeat the last
  // one: their dq is never written), lse2 / delta of each row (rows past the
  // padded length read its last one), keys each row sees
  const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + b * a.q_bs + h * a.q_hs;
  const __bf16* db = reinterpret_cast<const __bf16*>(a.dout) + b * a.q_bs + h * a.q_hs;
  bf16x8 q0r[KS], q1r[KS], d0r[KS], d1r[KS];
  const int r0 = min(qw0 + n, qlast), r1 = min(qw0 + 32 + n, qlast);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    q0r[s] = *reinterpret_cast<const bf16x8*>(qb + (int64_t)r0 * D + 16 * s + 8 * hh);
    q1r[s] = *reinterpret_cast<const bf16x8*>(qb + (int64_t)r1 * D + 16 * s + 8 * hh);
    d0r[s] = *reinterpret_cast<const bf16x8*>(db + (int64_t)r0 * D + 16 * s + 8 * hh);
    d1r[s] = *reinterpret_cast<const bf16x8*>(db + (int64_t)r1 * D + 16 * s + 8 * hh);
  }
  const int l0 = min(qw0 + n, a.Cqp - 1), l1 = min(qw0 + 32 + n, a.Cqp - 1);
  const float* lb = a.lse2 + b * a.l_bs + h * a.l_hs;
  const float* ndlb = a.ndelta + b * a.l_bs + h * a.l_hs;
  const float nl20 = -lb[l0], nl21 = -lb[l1];
  const float ndl0 = ndlb[l0], ndl1 = ndlb[l1];
  const int nal0 = a.causal ? allowed_prefix(a.kp, pos_of(a.qp, r0)) : a.Ck;
  const int nal1 = a.causal ? allowed_prefix(a.kp, pos_of(a.qp, r1)) : a.Ck;
  // first 32-key sub-tile with a key some row of the wave may not see (its
  // first row sees the fewest)
  const int first_mask =
      (a.causal ? allowed_prefix(a.kp, pos_of(a.qp, min(qw0, qlast))) : a.Ck) / 32;
  lds_loads_barrier();

  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto uni_ptr = [](const void* p) {
    const uint64_t v = (uint64_t)(size_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(size_t)(((uint64_t)hi << 32) | lo);
  };
  floatx16 dq0[DT], dq1[DT];
  dqw64::dq_loop(uni(n_kt), uni(first_mask), uni(lds_addr(Rows) + wk * 1024),
                 uni(lds_addr(Rows) + L::RBUF + wvv * 1024), uni(lds_addr(Kt) + wt * 1024),
                 uni(wk + NW * 4 < L::RINS), uni(wvv + NW * 4 < L::RINS), uni(wt + NW * 4 < L::TINS),
                 a.scale_log2, lds_addr(Rows) + kperm(n) * L::ROW + hh * 16,
                 lds_addr(Kt) + n * L::TROW + hh * 16, nl20, nl21, ndl0, ndl1, nal0 - 8 * hh,
                 nal1 - 8 * hh, uni_ptr(kb + (int64_t)min(2, n_kt - 1) * 64 * D),
                 uni_ptr(vb + (int64_t)min(2, n_kt - 1) * 64 * D),
                 uni_ptr(ktb + min(1, n_kt - 1) * 64), koff, voff, toff, q0r, q1r, d0r, d1r, dq0,
                 dq1);

  // add into the fp32 accumulators; lane holds query n of each block,
  // d = 32T + 8(i/4) + 4hh + i%4
  // All 32 loads of the old values (both blocks; rows past the block
  // re-read the last row and are not stored) go out before the first add,
  // so their latencies overlap.
  float* dqb = a.dq + b * a.dq_bs + h * a.dq_hs;
  float4 old[2][DT * 4];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float* row = dqb + (int64_t)min(qw0 + 32 * blk + n, qlast) * D;
#pragma unroll
    for (int j = 0; j < DT * 4; ++j)
      old[blk][j] = *reinterpret_cast<const float4*>(row + 32 * (j >> 2) + 8 * (j & 3) + 4 * hh);
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int qi = qw0 + 32 * blk + n;
    if (qi >= a.Cq) continue;
    floatx16(&dQt)[DT] = blk ? dq1 : dq0;
    float* dqr = dqb + (int64_t)qi * D;
#pragma unroll
    for (int T = 0; T < DT; ++T)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * T + 8 * q4 + 4 * hh;
        float4 x = old[blk][4 * T + q4];
        x.x += a.scale * dQt[T][4 * q4 + 0];
        x.y += a.scale * dQt[T][4 * q4 + 1];
        x.z += a.scale * dQt[T][4 * q4 + 2];
        x.w += a.scale * dQt[T][4 * q4 + 3];
        *reinterpret_cast<float4*>(dqr + d0) = x;
      }
  }
}

// ---------------------------------------------------------------------------
// -delta = -<dout, out> (stored negated: the dK / dV kernel starts its dP
// accumulation from it) and lse in exp2 units, per query row, padded.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* __restrict__ out,
                                                       const __bf16* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ lse2p,
                                                       float* __restrict__ ndeltap,
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
      ndeltap[row] = valid ? -acc : 0.f;
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
  return (size_t)2 * (2 * BwdLds<D>::RBUF) + (size_t)2 * (2 * BwdLds<D>::TBUF + 2048) +
         4 * kMaxHeads;
}
template <int D>
constexpr size_t dq_lds_bytes() {
  return (size_t)2 * (2 * BwdLds<D>::RBUF + BwdLds<D>::TBUF);
}

// The one-wave-per-SIMD dK / dV loop keeps a group's query heads one per
// lane (at most 64) and forms a tile's source addresses from 32-bit byte
// offsets (head * head stride + first query) added to the batch's base.
bool dkdv_w32_fits(const BwdArgs& a) {
  int ng_max = 0;
  for (int g = 0; g < a.Hkv; ++g) ng_max = std::max(ng_max, (int)(a.grp_off[g + 1] - a.grp_off[g]));
  const uint64_t h = (uint64_t)std::max(a.Hq - 1, 0), lim = 0xffffffffull;
  const uint64_t rows = h * (uint64_t)a.q_hs * 2 + (uint64_t)a.Cq * 256;
  const uint64_t trans = h * (uint64_t)a.qt_hs * 2 + (uint64_t)a.Cqp * 2;
  const uint64_t lse = h * (uint64_t)a.l_hs * 4 + (uint64_t)a.Cqp * 4;
  return ng_max <= 64 && (uint64_t)a.q_hs * 2 < (1ull << 31) && (uint64_t)a.qt_hs * 2 < (1ull << 31) &&
         (uint64_t)a.l_hs * 4 < (1ull << 31) && rows <= lim && trans <= lim && lse <= lim;
}

template <typename K>
hipError_t launch_big(K kern, size_t lds, int grid, const BwdArgs& a, hipStream_t s, int threads = 256) {
  static_assert(sizeof(BwdArgs) <= 4096, "kernel arguments");
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

void fill_bwd_heads(BwdArgs& a, int32_t Hq, int32_t Hkv, const std::vector<uint8_t>& kv_of,
                    const std::vector<uint8_t>& order) {
  memset(a.head_order, 0, sizeof a.head_order);
  memset(a.kv_of, 0, sizeof a.kv_of);
  memset(a.grp_off, 0, sizeof a.grp_off);
  for (int h = 0; h < Hq; ++h) {
    a.head_order[h] = order[h];
    a.kv_of[h] = kv_of[h];
  }
  std::vector<int> count(Hkv + 1, 0);
  for (int h = 0; h < Hq; ++h) count[kv_of[h] + 1]++;
  for (int g = 0; g < Hkv; ++g) count[g + 1] += count[g];
  for (int g = 0; g <= Hkv; ++g) a.grp_off[g] = (uint16_t)count[g];
}

hipError_t launch_bwd_dkdv(BwdArgs a, int D, hipStream_t s) {
  a.n_tiles = (a.Ck + 127) / 128;  // 128-key workgroups, per (batch, KV head)
  a.n_items = a.B * a.Hkv * a.n_tiles;
  a.per_xcd = (a.n_items + kXcds - 1) / kXcds;
  if (a.n_items <= 0) return hipSuccess;
  const int grid = a.per_xcd * kXcds;
  if (D == 128 && dkdv_w32_fits(a)) {
    if (a.Cq % 64 == 0) return launch_big(attn_bwd_dkdv_w32<false>, dkdv_w32_lds_bytes(), grid, a, s);
    return launch_big(attn_bwd_dkdv_w32<true>, dkdv_w32_lds_bytes(), grid, a, s);
  }
  if (D == 128) return launch_big(attn_bwd_dkdv<128>, dkdv_lds_bytes<128>(), grid, a, s);
  return launch_big(attn_bwd_dkdv<64>, dkdv_lds_bytes<64>(), grid, a, s);
}

hipError_t launch_bwd_dq(BwdArgs a, int D, hipStream_t s) {
  if (D == 128 && a.Ck % 64 == 0) {
    // whole 64-key tiles: the one-wave-per-SIMD kernel, 256 queries per workgroup
    a.n_tiles = (a.Cq + 64 * kDqW64Waves - 1) / (64 * kDqW64Waves);
    a.n_items = a.B * a.Hq * a.n_tiles;
    a.per_xcd = (a.n_items + kXcds - 1) / kXcds;
    if (a.n_items <= 0) return hipSuccess;
    return launch_big(attn_bwd_dq_w64, dq_w64_lds_bytes(), a.per_xcd * kXcds, a, s,
                      64 * kDqW64Waves);
  }
  constexpr int NW = kDqWaves;
  a.n_tiles = (a.Cq + 32 * NW - 1) / (32 * NW);  // 256-query workgroups, per (batch, query head)
  a.n_items = a.B * a.Hq * a.n_tiles;
  a.per_xcd = (a.n_items + kXcds - 1) / kXcds;
  if (a.n_items <= 0) return hipSuccess;
  const int grid = a.per_xcd * kXcds;
  if (D == 128) return launch_big(attn_bwd_dq<128>, dq_lds_bytes<128>(), grid, a, s, 64 * NW);
  return launch_big(attn_bwd_dq<64>, dq_lds_bytes<64>(), grid, a, s, 64 * NW);
}

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* lse2p,
                           float* ndeltap, int64_t BH, int64_t nblk, int64_t C, int64_t Cp, int D,
                           int64_t o_bh, int64_t l_bh, hipStream_t s) {
  const int64_t rows = BH * nblk * Cp;
  if (rows == 0) return hipSuccess;
  const int rows_per_block = 4 * (64 / (D / 8));
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  const __bf16* o = reinterpret_cast<const __bf16*>(out);
  const __bf16* d = reinterpret_cast<const __bf16*>(dout);
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, grid, dim3(256), 0, s, o, d, lse, lse2p, ndeltap, rows,
                       nblk, C, Cp, o_bh, l_bh);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, grid, dim3(256), 0, s, o, d, lse, lse2p, ndeltap, rows,
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
