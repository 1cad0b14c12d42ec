// Host side of the ring-attention library: the C ABI declared in
// include/ring_attn.h. Every entry point validates its arguments completely
// before it enqueues anything, then launches the gfx950 kernels.
//
// The virtual-ring driver follows "Context Parallelism" (aiwiki), the
// ring_attention listing (start the next hop, compute on the held block, wait,
// swap) and "Sequence Parallelism in Large Language Models ..." (llms.blog),
// "Algorithmic Mechanics" item 2 and the 4-GPU ring figure (at step k device
// i holds the block of source (i - k) mod N), with the point-to-point
// transfer replaced by an asynchronous device copy into a two-slot buffer.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <mutex>
#include <thread>
#include <vector>

#include "ra_internal.h"

using namespace ra;

namespace {

thread_local char g_err[512] = "";

ra_status fail(ra_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

ra_status hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define RA_HIP(call)                                       \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) return hip_fail(e_, #call);      \
  } while (0)

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline size_t esize(ra_dtype dt) { return dt == RA_BF16 ? 2 : 4; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Block positions as a PosDesc, with the validation rules of ra_pos.
ra_status make_pos(const ra_pos* p, int64_t rows, const char* name, PosDesc& out) {
  if (p == nullptr) {
    out = PosDesc{1, (int32_t)rows, 0, 0, 1};
    return RA_OK;
  }
  if (p->nseg != 1 && p->nseg != 2)
    return fail(RA_ERR_SHAPE, "%s.nseg must be 1 or 2 (got %d)", name, p->nseg);
  if (p->seg_len < 1 || p->nseg * p->seg_len != rows)
    return fail(RA_ERR_SHAPE, "%s: nseg*seg_len (%d*%lld) must equal the row count %lld", name,
                p->nseg, (long long)p->seg_len, (long long)rows);
  const int64_t stride = p->stride == 0 ? 1 : p->stride;
  if (stride < 1 || stride > INT32_MAX)
    return fail(RA_ERR_SHAPE, "%s.stride must be in [1, 2^31-1] (got %lld)", name,
                (long long)p->stride);
  if (p->start[0] < 0) return fail(RA_ERR_SHAPE, "%s.start[0] must be >= 0", name);
  const int64_t span = (p->seg_len - 1) * stride;  // seg_len < 2^31 here (row count check)
  if (p->start[0] > INT32_MAX || span > INT32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "%s: positions beyond 2^31-1", name);
  if (p->nseg == 2 && p->start[1] <= p->start[0] + span)
    return fail(RA_ERR_SHAPE, "%s: start[1] must exceed start[0] + (seg_len-1)*stride", name);
  const int64_t last = p->start[p->nseg - 1] + span;
  if (last > INT32_MAX) return fail(RA_ERR_UNSUPPORTED, "%s: positions beyond 2^31-1", name);
  out = PosDesc{p->nseg, (int32_t)p->seg_len, (int32_t)p->start[0],
                (int32_t)(p->nseg == 2 ? p->start[1] : 0), (int32_t)stride};
  return RA_OK;
}

// floor(a / b) for b > 0
inline int64_t floordiv(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Allowed (query, key) pairs between two position descriptors (per head).
int64_t pairs_segment(int64_t a, int64_t La, int64_t b, int64_t Lb) {
  // sum over i in [0, La) of clamp(a + i - b + 1, 0, Lb)
  const int64_t x0 = a - b + 1;
  int64_t total = 0;
  // i where x0 + i >= Lb contributes Lb
  int64_t i_full = std::max<int64_t>(0, Lb - x0);  // first i with x0+i >= Lb
  int64_t i_pos = std::max<int64_t>(0, 1 - x0);    // first i with x0+i >= 1
  i_full = std::min(i_full, La);
  i_pos = std::min(i_pos, La);
  if (i_full > i_pos) {
    const int64_t n = i_full - i_pos;
    const int64_t first = x0 + i_pos;
    total += n * first + n * (n - 1) / 2;
  }
  total += (La - std::max(i_full, i_pos)) * Lb;
  return total;
}

int64_t pairs_between(const PosDesc& q, int64_t Cq, const PosDesc& k, int64_t Ck, bool causal) {
  if (!causal) return Cq * Ck;
  int64_t total = 0;
  for (int sq = 0; sq < q.nseg; ++sq)
    for (int sk = 0; sk < k.nseg; ++sk) {
      const int64_t a = sq == 0 ? q.start0 : q.start1, La = q.nseg == 1 ? Cq : q.seg;
      const int64_t b = sk == 0 ? k.start0 : k.start1, Lb = k.nseg == 1 ? Ck : k.seg;
      if (q.stride == k.stride) {
        // key j <= query i  <=>  j <= i + floor((a - b) / stride)
        total += pairs_segment(floordiv(a - b, q.stride), La, 0, Lb);
      } else {
        for (int64_t i = 0; i < La; ++i)
          total += std::clamp<int64_t>(floordiv(a + i * q.stride - b, k.stride) + 1, 0, Lb);
      }
    }
  return total;
}

// ---------------------------------------------------------------- timing
struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> ev;  // pairs: start, stop
  size_t used = 0;             // pairs recorded since the last read
  int64_t launches = 0;
  double flops = 0.0;
};
Timing g_timing;
constexpr size_t kMaxTimed = 65536;
constexpr size_t kPreTimed = 4096;  // launch event pairs created when timing is enabled
// The timing events only time: no memory has to become visible when they are
// recorded, so they skip the system-scope release and acquire (cache
// writeback and invalidation) a default event performs around every launch.
constexpr unsigned kTimingEventFlags = hipEventDisableSystemFence;

// Launch an attention kernel (forward or backward), bracketed by timing events
// when enabled; `flops` is its useful work.
template <class F>
ra_status timed(hipStream_t s, double flops, F&& launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.enabled) {
      g_timing.launches++;
      g_timing.flops += flops;
      if (g_timing.used < kMaxTimed) {
        if (2 * g_timing.used + 2 > g_timing.ev.size()) {
          for (int i = 0; i < 256; ++i) {
            hipEvent_t e;
            RA_HIP(hipEventCreateWithFlags(&e, kTimingEventFlags));
            g_timing.ev.push_back(e);
          }
        }
        e0 = g_timing.ev[2 * g_timing.used];
        e1 = g_timing.ev[2 * g_timing.used + 1];
        g_timing.used++;
      }
    }
  }
  if (e0) RA_HIP(hipEventRecord(e0, s));
  hipError_t e = launch();
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  if (e1) RA_HIP(hipEventRecord(e1, s));
  return RA_OK;
}

ra_status timed_launch(const AttnArgs& a, ra_dtype dt, int D, hipStream_t s, double flops) {
  return timed(s, flops, [&] { return launch_attn(a, dt, D, s); });
}

// ---------------------------------------------------------------- ring events
// The ready / freed / V^T-done events of ONE ring call. Every call creates
// its own set and destroys it after enqueueing (a destroyed event that work
// still waits on completes normally), so calls from several host threads
// never bind a wait to another call's record and the library keeps no
// per-device state between calls.
struct RingEvents {
  hipEvent_t ready[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr}, vt_done = nullptr;
  ~RingEvents() {
    for (hipEvent_t e : {ready[0], ready[1], freed[0], freed[1], vt_done})
      if (e) (void)hipEventDestroy(e);
  }
  ra_status create() {
    for (int i = 0; i < 2; ++i) {
      RA_HIP(hipEventCreateWithFlags(&ready[i], hipEventDisableTiming));
      RA_HIP(hipEventCreateWithFlags(&freed[i], hipEventDisableTiming));
    }
    RA_HIP(hipEventCreateWithFlags(&vt_done, hipEventDisableTiming));
    return RA_OK;
  }
};

// ---------------------------------------------------------------- shared checks
ra_status check_common(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, ra_dtype dt,
                       const int32_t* kv_map, float scale, std::vector<uint8_t>& kv_of,
                       std::vector<uint8_t>& order) {
  if (dt != RA_BF16 && dt != RA_F32) return fail(RA_ERR_DTYPE, "unknown dtype %d", (int)dt);
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(RA_ERR_SHAPE, "B, Hq, Hkv must be >= 1 (got %d, %d, %d)", B, Hq, Hkv);
  if (D != 64 && D != 128) return fail(RA_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", D);
  if (Hq > kMaxHeads || Hkv > kMaxHeads)
    return fail(RA_ERR_UNSUPPORTED, "more than %d heads", kMaxHeads);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(RA_ERR_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  kv_of.assign(Hq, 0);
  if (kv_map == nullptr) {
    if (Hq % Hkv) return fail(RA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    for (int h = 0; h < Hq; ++h) kv_of[h] = (uint8_t)(h / (Hq / Hkv));
  } else {
    for (int h = 0; h < Hq; ++h) {
      if (kv_map[h] < 0 || kv_map[h] >= Hkv)
        return fail(RA_ERR_SHAPE, "kv_head_of_q[%d]=%d outside [0, %d)", h, kv_map[h], Hkv);
      kv_of[h] = (uint8_t)kv_map[h];
    }
  }
  // query heads ordered by KV head (stable), so heads sharing K/V are adjacent
  order.resize(Hq);
  for (int h = 0; h < Hq; ++h) order[h] = (uint8_t)h;
  std::stable_sort(order.begin(), order.end(),
                   [&](uint8_t x, uint8_t y) { return kv_of[x] < kv_of[y]; });
  return RA_OK;
}

}  // namespace

// ============================================================================
extern "C" {

const char* ra_status_str(ra_status s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_ERR_NULL: return "RA_ERR_NULL";
    case RA_ERR_SHAPE: return "RA_ERR_SHAPE";
    case RA_ERR_DTYPE: return "RA_ERR_DTYPE";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_ALIGN: return "RA_ERR_ALIGN";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE";
    case RA_ERR_ARG: return "RA_ERR_ARG";
    case RA_ERR_HIP: return "RA_ERR_HIP";
    case RA_ERR_TIMEOUT: return "RA_ERR_TIMEOUT";
  }
  return "RA_ERR_UNKNOWN";
}

const char* ra_last_error(void) { return g_err; }

size_t ra_block_attn_workspace_bytes(int32_t B, int32_t Hkv, int64_t Ck, int32_t D,
                                     ra_dtype dtype) {
  if (dtype != RA_BF16 || B < 1 || Hkv < 1 || Ck < 1 || D < 1) return 0;
  return (size_t)B * Hkv * D * round_up(Ck, kVtAlign) * 2;
}

ra_status ra_block_attn_fwd(const void* q, const void* k, const void* v, float* out, float* lse,
                            int32_t B, int32_t Hq, int32_t Hkv, int64_t Cq, int64_t Ck, int32_t D,
                            ra_dtype dtype, const ra_pos* q_pos, const ra_pos* k_pos,
                            const int32_t* kv_head_of_q, int32_t causal, float scale,
                            int32_t accumulate, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_err[0] = 0;
  std::vector<uint8_t> kv_of, order;
  ra_status st = check_common(B, Hq, Hkv, D, dtype, kv_head_of_q, scale, kv_of, order);
  if (st != RA_OK) return st;
  if (Cq < 0 || Ck < 0) return fail(RA_ERR_SHAPE, "negative row count");
  if (Cq > INT32_MAX || Ck > INT32_MAX) return fail(RA_ERR_UNSUPPORTED, "block rows beyond 2^31-1");
  if ((causal != 0 && causal != 1) || (accumulate != 0 && accumulate != 1))
    return fail(RA_ERR_ARG, "causal and accumulate must be 0 or 1");
  if (Cq == 0) return RA_OK;
  if (!q || !out || !lse) return fail(RA_ERR_NULL, "q, out and lse must not be NULL");
  if (Ck > 0 && (!k || !v)) return fail(RA_ERR_NULL, "k and v must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16) || (Ck > 0 && (!aligned(k, 16) || !aligned(v, 16))))
    return fail(RA_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  PosDesc qp, kp;
  if ((st = make_pos(q_pos, Cq, "q_pos", qp)) != RA_OK) return st;
  if (Ck > 0) {
    if ((st = make_pos(k_pos, Ck, "k_pos", kp)) != RA_OK) return st;
  } else {
    kp = PosDesc{1, 0, 0, 0, 1};
  }
  const size_t need = ra_block_attn_workspace_bytes(B, Hkv, Ck, D, dtype);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need,
                  workspace_bytes);
    if (!aligned(workspace, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.run_out = out;
  a.run_lse = lse;
  a.q_bs = (int64_t)Hq * Cq * D;
  a.q_hs = Cq * D;
  a.k_bs = (int64_t)Hkv * Ck * D;
  a.k_hs = Ck * D;
  a.ro_bs = a.q_bs;
  a.ro_hs = a.q_hs;
  a.rl_bs = (int64_t)Hq * Cq;
  a.rl_hs = Cq;
  a.Cq = (int32_t)Cq;
  a.Ck = (int32_t)Ck;
  a.qp = qp;
  a.kp = kp;
  a.causal = causal;
  a.accumulate = accumulate;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (dtype == RA_BF16 && Ck > 0) {
    const int64_t Cpad = round_up(Ck, kVtAlign);
    hipError_t e = launch_vt_transpose(v, workspace, (int64_t)B * Hkv, 1, Ck, Cpad, D, Ck * D, s);
    if (e != hipSuccess) return hip_fail(e, "V transpose launch");
    a.v = workspace;
    a.v_bs = (int64_t)Hkv * D * Cpad;
    a.v_hs = (int64_t)D * Cpad;
    a.v_ld = Cpad;
  } else {
    a.v = v;
    a.v_bs = a.k_bs;
    a.v_hs = a.k_hs;
    a.v_ld = D;
  }
  fill_attn_work(a, dtype, B, Hq, Cq, kv_of, order);
  const double flops = 4.0 * D * B * Hq * (double)(Ck > 0 ? pairs_between(qp, Cq, kp, Ck, causal) : 0);
  return timed_launch(a, dtype, D, s, flops);
}

ra_status ra_block_attn_fwd_noalloc(const void* q, const void* k, const void* v, float* out,
                                    float* lse, int32_t B, int32_t Hq, int32_t Hkv, int64_t Cq,
                                    int64_t Ck, int32_t D, ra_dtype dtype, const ra_pos* q_pos,
                                    const ra_pos* k_pos, const int32_t* kv_head_of_q,
                                    int32_t causal, float scale, int32_t accumulate,
                                    void* stream) {
  g_err[0] = 0;
  const size_t need = ra_block_attn_workspace_bytes(B, Hkv, Ck, D, dtype);
  if (need > kNoAllocScratchBytes)
    return fail(RA_ERR_WORKSPACE,
                "the transposed V block needs %zu bytes, beyond the %zu-byte static scratch "
                "(B*Hkv*D*round_up(Ck, 64)*2 must not exceed it)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
  }
  return ra_block_attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Cq, Ck, D, dtype, q_pos, k_pos,
                           kv_head_of_q, causal, scale, accumulate, ws,
                           need > 0 ? kNoAllocScratchBytes : 0, stream);
}

ra_status ra_lse_merge(float* out, float* lse, const float* out_b, const float* lse_b,
                       int64_t rows, int32_t D, void* stream) {
  g_err[0] = 0;
  if (rows < 0 || D < 1) return fail(RA_ERR_SHAPE, "rows must be >= 0 and D >= 1");
  if (rows == 0) return RA_OK;
  if (!out || !lse || !out_b || !lse_b) return fail(RA_ERR_NULL, "NULL pointer");
  if (!aligned(out, 4) || !aligned(lse, 4) || !aligned(out_b, 4) || !aligned(lse_b, 4))
    return fail(RA_ERR_ALIGN, "float arrays must be 4-byte aligned");
  hipError_t e = launch_lse_merge(out, lse, out_b, lse_b, rows, D, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "lse merge launch");
  return RA_OK;
}

ra_status ra_zigzag_permute(const void* src, void* dst, int64_t outer, int64_t S, int64_t row_bytes,
                            int32_t N, int32_t inverse, void* stream) {
  g_err[0] = 0;
  if (N < 1) return fail(RA_ERR_SHAPE, "N must be >= 1");
  if (outer < 0 || S < 0 || row_bytes < 1) return fail(RA_ERR_SHAPE, "bad sizes");
  if (S % (2 * (int64_t)N)) return fail(RA_ERR_SHAPE, "S=%lld not divisible by 2N=%d", (long long)S, 2 * N);
  if (inverse != 0 && inverse != 1) return fail(RA_ERR_ARG, "inverse must be 0 or 1");
  if (outer == 0 || S == 0) return RA_OK;
  if (!src || !dst) return fail(RA_ERR_NULL, "NULL pointer");
  const uintptr_t bytes = (uintptr_t)outer * S * row_bytes;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RA_ERR_ARG, "src and dst overlap");
  hipError_t e = launch_zigzag_permute(src, dst, outer, S, row_bytes, N, inverse,
                                       reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  return RA_OK;
}

ra_status ra_striped_permute(const void* src, void* dst, int64_t outer, int64_t S, int64_t row_bytes,
                             int32_t N, int32_t inverse, void* stream) {
  g_err[0] = 0;
  if (N < 1) return fail(RA_ERR_SHAPE, "N must be >= 1");
  if (outer < 0 || S < 0 || row_bytes < 1) return fail(RA_ERR_SHAPE, "bad sizes");
  if (S % N) return fail(RA_ERR_SHAPE, "S=%lld not divisible by N=%d", (long long)S, N);
  if (inverse != 0 && inverse != 1) return fail(RA_ERR_ARG, "inverse must be 0 or 1");
  if (outer == 0 || S == 0) return RA_OK;
  if (!src || !dst) return fail(RA_ERR_NULL, "NULL pointer");
  const uintptr_t bytes = (uintptr_t)outer * S * row_bytes;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RA_ERR_ARG, "src and dst overlap");
  hipError_t e = launch_striped_permute(src, dst, outer, S, row_bytes, N, inverse,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  return RA_OK;
}

// Workspace of the ring: [V^T home blocks (bf16)] [2 KV slots] [fp32 running out]
namespace {
struct RingLayout {
  int64_t C, Cpad;
  size_t vt_home, slot_k, slot_v, slot, acc, total;
};
RingLayout ring_layout(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D, ra_dtype dt,
                       int32_t N) {
  RingLayout L{};
  L.C = S / N;
  L.Cpad = round_up(L.C, kVtAlign);
  const size_t es = esize(dt);
  auto up = [](size_t x) { return (size_t)round_up((int64_t)x, 256); };
  L.vt_home = dt == RA_BF16 ? up((size_t)B * Hkv * N * D * L.Cpad * es) : 0;
  L.slot_k = up((size_t)B * Hkv * L.C * D * es);
  L.slot_v = dt == RA_BF16 ? up((size_t)B * Hkv * D * L.Cpad * es) : L.slot_k;
  L.slot = L.slot_k + L.slot_v;
  L.acc = up((size_t)B * Hq * L.C * D * 4);
  L.total = L.vt_home + 2 * L.slot + L.acc;
  return L;
}
}  // namespace

size_t ra_ring_sim_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                   ra_dtype dtype, int32_t N) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || N < 1 || D < 1 || S % N) return 0;
  if (dtype != RA_BF16 && dtype != RA_F32) return 0;
  return ring_layout(B, Hq, Hkv, S, D, dtype, N).total;
}

ra_status ra_ring_sim_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                          ra_dtype dtype, int32_t N, ra_layout layout, int32_t causal,
                          float scale, const int32_t* kv_head_of_q, void* workspace,
                          size_t workspace_bytes, void* compute_stream, void* copy_stream) {
  g_err[0] = 0;
  std::vector<uint8_t> kv_of, order;
  ra_status st = check_common(B, Hq, Hkv, D, dtype, kv_head_of_q, scale, kv_of, order);
  if (st != RA_OK) return st;
  if (layout != RA_CONTIGUOUS && layout != RA_ZIGZAG && layout != RA_STRIPED)
    return fail(RA_ERR_ARG, "unknown layout");
  if (causal != 0 && causal != 1) return fail(RA_ERR_ARG, "causal must be 0 or 1");
  if (N < 1) return fail(RA_ERR_SHAPE, "N must be >= 1");
  if (S < 0) return fail(RA_ERR_SHAPE, "S must be >= 0");
  const int64_t div = layout == RA_ZIGZAG ? 2 * (int64_t)N : N;
  if (S % div) return fail(RA_ERR_SHAPE, "S=%lld not divisible by %lld", (long long)S, (long long)div);
  if (S == 0) return RA_OK;
  if (S > INT32_MAX) return fail(RA_ERR_UNSUPPORTED, "S beyond 2^31-1");
  if (!q || !k || !v || !out || !lse) return fail(RA_ERR_NULL, "NULL tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(RA_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  const RingLayout L = ring_layout(B, Hq, Hkv, S, D, dtype, N);
  if (!workspace || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", L.total, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");

  hipStream_t cs = reinterpret_cast<hipStream_t>(compute_stream);
  hipStream_t xs = copy_stream ? reinterpret_cast<hipStream_t>(copy_stream) : cs;
  RingEvents ring_ev;
  RingEvents* ev = &ring_ev;
  if (xs != cs && (st = ring_ev.create()) != RA_OK) return st;
  const size_t es = esize(dtype);
  const int64_t C = L.C, Cpad = L.Cpad;
  char* ws = reinterpret_cast<char*>(workspace);
  char* vt_home = ws;
  char* slot[2] = {ws + L.vt_home, ws + L.vt_home + L.slot};
  float* acc = reinterpret_cast<float*>(ws + L.vt_home + 2 * L.slot);
  const bool bf16 = dtype == RA_BF16;

  // V^T home blocks, once per call: [B*Hkv][N][D][Cpad].
  if (bf16) {
    hipError_t e = launch_vt_transpose(v, vt_home, (int64_t)B * Hkv, N, C, Cpad, D, S * D, cs);
    if (e != hipSuccess) return hip_fail(e, "V transpose launch");
  }
  if (xs != cs) {
    RA_HIP(hipEventRecord(ev->vt_done, cs));
    RA_HIP(hipStreamWaitEvent(xs, ev->vt_done, 0));
  }

  auto pos_of_rank = [&](int r) {
    PosDesc p;
    if (layout == RA_ZIGZAG) {
      const int64_t c = S / (2 * N);
      p = PosDesc{2, (int32_t)c, (int32_t)(r * c), (int32_t)((2 * N - 1 - r) * c), 1};
    } else if (layout == RA_STRIPED) {
      p = PosDesc{1, (int32_t)C, (int32_t)r, 0, (int32_t)N};
    } else {
      p = PosDesc{1, (int32_t)C, (int32_t)(r * C), 0, 1};
    }
    return p;
  };
  // Enqueue the copy of source rank `src`'s K and V blocks into slot `sl`.
  auto copy_block = [&](int src, int sl) -> ra_status {
    const size_t row_k = (size_t)C * D * es;
    RA_HIP(hipMemcpy2DAsync(slot[sl], row_k, (const char*)k + (size_t)src * row_k, (size_t)S * D * es,
                            row_k, (size_t)B * Hkv, hipMemcpyDeviceToDevice, xs));
    char* sv = slot[sl] + L.slot_k;
    if (bf16) {
      const size_t blk = (size_t)D * Cpad * es;
      RA_HIP(hipMemcpy2DAsync(sv, blk, vt_home + (size_t)src * blk, (size_t)N * blk, blk,
                              (size_t)B * Hkv, hipMemcpyDeviceToDevice, xs));
    } else {
      RA_HIP(hipMemcpy2DAsync(sv, row_k, (const char*)v + (size_t)src * row_k, (size_t)S * D * es,
                              row_k, (size_t)B * Hkv, hipMemcpyDeviceToDevice, xs));
    }
    return RA_OK;
  };

  for (int r = 0; r < N; ++r) {
    const PosDesc qp = pos_of_rank(r);
    for (int step = 0; step < N; ++step) {
      const int src = ((r - step) % N + N) % N;
      // Start the next hop before computing on the held block.
      if (step + 1 < N) {
        const int nsrc = ((r - step - 1) % N + N) % N;
        const int sl = (step + 1) & 1;
        if (xs != cs) RA_HIP(hipStreamWaitEvent(xs, ev->freed[sl], 0));
        if ((st = copy_block(nsrc, sl)) != RA_OK) return st;
        if (xs != cs) RA_HIP(hipEventRecord(ev->ready[sl], xs));
      }
      AttnArgs a;
      memset(&a, 0, sizeof a);
      a.q = (const char*)q + (size_t)r * C * D * es;
      a.q_bs = (int64_t)Hq * S * D;
      a.q_hs = S * D;
      if (step == 0) {  // the rank's own block, read in place
        a.k = (const char*)k + (size_t)r * C * D * es;
        a.k_bs = (int64_t)Hkv * S * D;
        a.k_hs = S * D;
        if (bf16) {
          a.v = vt_home + (size_t)r * D * Cpad * es;
          a.v_bs = (int64_t)Hkv * N * D * Cpad;
          a.v_hs = (int64_t)N * D * Cpad;
          a.v_ld = Cpad;
        } else {
          a.v = (const char*)v + (size_t)r * C * D * es;
          a.v_bs = a.k_bs;
          a.v_hs = a.k_hs;
          a.v_ld = D;
        }
      } else {
        const int sl = step & 1;
        if (xs != cs) RA_HIP(hipStreamWaitEvent(cs, ev->ready[sl], 0));
        a.k = slot[sl];
        a.k_bs = (int64_t)Hkv * C * D;
        a.k_hs = C * D;
        a.v = slot[sl] + L.slot_k;
        if (bf16) {
          a.v_bs = (int64_t)Hkv * D * Cpad;
          a.v_hs = (int64_t)D * Cpad;
          a.v_ld = Cpad;
        } else {
          a.v_bs = a.k_bs;
          a.v_hs = a.k_hs;
          a.v_ld = D;
        }
      }
      a.run_out = acc;
      a.ro_bs = (int64_t)Hq * C * D;
      a.ro_hs = C * D;
      a.run_lse = lse + (size_t)r * C;  // the lse output doubles as running lse
      a.rl_bs = (int64_t)Hq * S;
      a.rl_hs = S;
      if (step == N - 1) {
        a.fin_out = (char*)out + (size_t)r * C * D * es;
        a.fo_bs = (int64_t)Hq * S * D;
        a.fo_hs = S * D;
        a.fin_lse = lse + (size_t)r * C;
        a.fl_bs = a.rl_bs;
        a.fl_hs = a.rl_hs;
      }
      a.Cq = (int32_t)C;
      a.Ck = (int32_t)C;
      a.qp = qp;
      a.kp = pos_of_rank(src);
      a.causal = causal;
      a.accumulate = step > 0;
      a.scale = scale;
      a.scale_log2 = scale * 1.4426950408889634f;
      fill_attn_work(a, dtype, B, Hq, C, kv_of, order);
      const double flops = 4.0 * D * B * Hq * (double)pairs_between(a.qp, C, a.kp, C, causal);
      if ((st = timed_launch(a, dtype, D, cs, flops)) != RA_OK) return st;
      if (step > 0 && xs != cs) RA_HIP(hipEventRecord(ev->freed[step & 1], cs));
    }
  }
  return RA_OK;
}

// ---------------------------------------------------------------- backward
namespace {
struct BwdLayout {
  int64_t Cqp, Ckp;
  size_t qt, dot, kt, lse2, delta, total;  // byte offsets / total
};
// [Q^T][dO^T][K^T][lse2][delta] for nq query slabs of Cq rows and nk key slabs of Ck
BwdLayout bwd_layout(int64_t BHq, int64_t BHkv, int64_t nblk, int64_t Cq, int64_t Ck, int32_t D) {
  auto up = [](size_t x) { return (size_t)round_up((int64_t)x, 256); };
  BwdLayout L{};
  L.Cqp = round_up(Cq, kBwdRowPad);
  L.Ckp = round_up(Ck, kBwdRowPad);
  const size_t tq = up((size_t)BHq * nblk * D * L.Cqp * 2);
  const size_t tk = up((size_t)BHkv * nblk * D * L.Ckp * 2);
  const size_t rv = up((size_t)BHq * nblk * L.Cqp * 4);
  L.qt = 0;
  L.dot = tq;
  L.kt = 2 * tq;
  L.lse2 = 2 * tq + tk;
  L.delta = L.lse2 + rv;
  L.total = L.delta + rv;
  return L;
}

ra_status check_bwd(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, ra_dtype dt,
                    const int32_t* kv_map, float scale, std::vector<uint8_t>& kv_of,
                    std::vector<uint8_t>& order) {
  ra_status st = check_common(B, Hq, Hkv, D, dt, kv_map, scale, kv_of, order);
  if (st != RA_OK) return st;
  if (dt != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "the backward supports bf16 inputs only");
  return RA_OK;
}

// Work decomposition and head tables of both backward kernels.
ra_status launch_bwd_pair(BwdArgs a, int32_t D, hipStream_t s) {
  const double pairs = (double)(a.Ck > 0 ? pairs_between(a.qp, a.Cq, a.kp, a.Ck, a.causal) : 0);
  if (a.Cq == 0 || a.Ck == 0) return RA_OK;
  const double fl = (double)D * a.B * a.Hq * pairs;
  ra_status st = timed(s, 8.0 * fl, [&] { return launch_bwd_dkdv(a, D, s); });
  if (st != RA_OK) return st;
  return timed(s, 2.0 * fl, [&] { return launch_bwd_dq(a, D, s); });
}
}  // namespace

size_t ra_block_attn_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t Cq,
                                         int64_t Ck, int32_t D, ra_dtype dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Cq < 0 || Ck < 0 || D < 1 || dtype != RA_BF16) return 0;
  return bwd_layout((int64_t)B * Hq, (int64_t)B * Hkv, 1, Cq, Ck, D).total;
}

ra_status ra_block_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, float* dq, float* dk, float* dv,
                            int32_t B, int32_t Hq, int32_t Hkv, int64_t Cq, int64_t Ck, int32_t D,
                            ra_dtype dtype, const ra_pos* q_pos, const ra_pos* k_pos,
                            const int32_t* kv_head_of_q, int32_t causal, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  std::vector<uint8_t> kv_of, order;
  ra_status st = check_bwd(B, Hq, Hkv, D, dtype, kv_head_of_q, scale, kv_of, order);
  if (st != RA_OK) return st;
  if (Cq < 0 || Ck < 0) return fail(RA_ERR_SHAPE, "negative row count");
  if (Cq > INT32_MAX || Ck > INT32_MAX) return fail(RA_ERR_UNSUPPORTED, "block rows beyond 2^31-1");
  if (causal != 0 && causal != 1) return fail(RA_ERR_ARG, "causal must be 0 or 1");
  if (Cq == 0 || Ck == 0) return RA_OK;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(RA_ERR_NULL, "NULL tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(RA_ERR_ALIGN, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  PosDesc qp, kp;
  if ((st = make_pos(q_pos, Cq, "q_pos", qp)) != RA_OK) return st;
  if ((st = make_pos(k_pos, Ck, "k_pos", kp)) != RA_OK) return st;
  const BwdLayout L = bwd_layout((int64_t)B * Hq, (int64_t)B * Hkv, 1, Cq, Ck, D);
  if (!workspace || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", L.total, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  hipError_t e;
  if ((e = launch_vt_transpose(q, ws + L.qt, (int64_t)B * Hq, 1, Cq, L.Cqp, D, Cq * D, s)) != hipSuccess ||
      (e = launch_vt_transpose(dout, ws + L.dot, (int64_t)B * Hq, 1, Cq, L.Cqp, D, Cq * D, s)) != hipSuccess ||
      (e = launch_vt_transpose(k, ws + L.kt, (int64_t)B * Hkv, 1, Ck, L.Ckp, D, Ck * D, s)) != hipSuccess ||
      (e = launch_bwd_prep(out, dout, lse, (float*)(ws + L.lse2), (float*)(ws + L.delta),
                           (int64_t)B * Hq, 1, Cq, L.Cqp, D, Cq * D, Cq, s)) != hipSuccess)
    return hip_fail(e, "backward preparation launch");
  BwdArgs a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.qt = ws + L.qt; a.dot = ws + L.dot; a.kt = ws + L.kt;
  a.lse2 = (const float*)(ws + L.lse2); a.ndelta = (const float*)(ws + L.delta);
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.q_hs = Cq * D;            a.q_bs = (int64_t)Hq * a.q_hs;
  a.k_hs = Ck * D;            a.k_bs = (int64_t)Hkv * a.k_hs;
  a.qt_hs = (int64_t)D * L.Cqp; a.qt_bs = (int64_t)Hq * a.qt_hs;
  a.kt_hs = (int64_t)D * L.Ckp; a.kt_bs = (int64_t)Hkv * a.kt_hs;
  a.l_hs = L.Cqp;             a.l_bs = (int64_t)Hq * a.l_hs;
  a.dq_hs = a.q_hs;           a.dq_bs = a.q_bs;
  a.dk_hs = a.k_hs;           a.dk_bs = a.k_bs;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  a.Cq = (int32_t)Cq; a.Ck = (int32_t)Ck;
  a.Cqp = (int32_t)L.Cqp; a.Ckp = (int32_t)L.Ckp;
  a.qp = qp; a.kp = kp;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  fill_bwd_heads(a, Hq, Hkv, kv_of, order);
  return launch_bwd_pair(a, D, s);
}

namespace {
// [fp32 dq][fp32 dk][fp32 dv] [Q^T, dO^T, K^T, lse2, delta of all N blocks]
struct RingBwdLayout {
  int64_t C;
  size_t dq, dk, dv, prep, total;
  BwdLayout P;
};
RingBwdLayout ring_bwd_layout(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                              int32_t N) {
  auto up = [](size_t x) { return (size_t)round_up((int64_t)x, 256); };
  RingBwdLayout L{};
  L.C = S / N;
  L.dq = 0;
  L.dk = up((size_t)B * Hq * S * D * 4);
  L.dv = L.dk + up((size_t)B * Hkv * S * D * 4);
  L.prep = L.dv + up((size_t)B * Hkv * S * D * 4);
  L.P = bwd_layout((int64_t)B * Hq, (int64_t)B * Hkv, N, L.C, L.C, D);
  L.total = L.prep + L.P.total;
  return L;
}
}  // namespace

size_t ra_ring_sim_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                       ra_dtype dtype, int32_t N) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || N < 1 || D < 1 || S % N || dtype != RA_BF16) return 0;
  return ring_bwd_layout(B, Hq, Hkv, S, D, N).total;
}

ra_status ra_ring_sim_bwd(const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                          ra_dtype dtype, int32_t N, ra_layout layout, int32_t causal,
                          float scale, const int32_t* kv_head_of_q, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  std::vector<uint8_t> kv_of, order;
  ra_status st = check_bwd(B, Hq, Hkv, D, dtype, kv_head_of_q, scale, kv_of, order);
  if (st != RA_OK) return st;
  if (layout != RA_CONTIGUOUS && layout != RA_ZIGZAG && layout != RA_STRIPED)
    return fail(RA_ERR_ARG, "unknown layout");
  if (causal != 0 && causal != 1) return fail(RA_ERR_ARG, "causal must be 0 or 1");
  if (N < 1) return fail(RA_ERR_SHAPE, "N must be >= 1");
  if (S < 0) return fail(RA_ERR_SHAPE, "S must be >= 0");
  const int64_t div = layout == RA_ZIGZAG ? 2 * (int64_t)N : N;
  if (S % div) return fail(RA_ERR_SHAPE, "S=%lld not divisible by %lld", (long long)S, (long long)div);
  if (S == 0) return RA_OK;
  if (S > INT32_MAX) return fail(RA_ERR_UNSUPPORTED, "S beyond 2^31-1");
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(RA_ERR_NULL, "NULL tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(RA_ERR_ALIGN, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  const RingBwdLayout L = ring_bwd_layout(B, Hq, Hkv, S, D, N);
  if (!workspace || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", L.total, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  const int64_t C = L.C, Cp = L.P.Cqp;
  float* dq_acc = reinterpret_cast<float*>(ws + L.dq);
  float* dk_acc = reinterpret_cast<float*>(ws + L.dk);
  float* dv_acc = reinterpret_cast<float*>(ws + L.dv);
  char* pw = ws + L.prep;
  hipError_t e;
  if ((e = launch_zero_fill(ws, L.prep, s)) != hipSuccess) return hip_fail(e, "accumulator clear");
  if ((e = launch_vt_transpose(q, pw + L.P.qt, (int64_t)B * Hq, N, C, Cp, D, S * D, s)) != hipSuccess ||
      (e = launch_vt_transpose(dout, pw + L.P.dot, (int64_t)B * Hq, N, C, Cp, D, S * D, s)) != hipSuccess ||
      (e = launch_vt_transpose(k, pw + L.P.kt, (int64_t)B * Hkv, N, C, Cp, D, S * D, s)) != hipSuccess ||
      (e = launch_bwd_prep(out, dout, lse, (float*)(pw + L.P.lse2), (float*)(pw + L.P.delta),
                           (int64_t)B * Hq, N, C, Cp, D, S * D, S, s)) != hipSuccess)
    return hip_fail(e, "backward preparation launch");

  auto pos_of_rank = [&](int r) {
    if (layout == RA_ZIGZAG) {
      const int64_t c = S / (2 * N);
      return PosDesc{2, (int32_t)c, (int32_t)(r * c), (int32_t)((2 * N - 1 - r) * c), 1};
    }
    if (layout == RA_STRIPED) return PosDesc{1, (int32_t)C, (int32_t)r, 0, (int32_t)N};
    return PosDesc{1, (int32_t)C, (int32_t)(r * C), 0, 1};
  };
  BwdArgs a;
  memset(&a, 0, sizeof a);
  a.q_hs = S * D;              a.q_bs = (int64_t)Hq * a.q_hs;
  a.k_hs = S * D;              a.k_bs = (int64_t)Hkv * a.k_hs;
  a.qt_hs = (int64_t)N * D * Cp; a.qt_bs = (int64_t)Hq * a.qt_hs;
  a.kt_hs = (int64_t)N * D * Cp; a.kt_bs = (int64_t)Hkv * a.kt_hs;
  a.l_hs = (int64_t)N * Cp;    a.l_bs = (int64_t)Hq * a.l_hs;
  a.dq_hs = a.q_hs;            a.dq_bs = a.q_bs;
  a.dk_hs = a.k_hs;            a.dk_bs = a.k_bs;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  a.Cq = a.Ck = (int32_t)C;
  a.Cqp = a.Ckp = (int32_t)Cp;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  fill_bwd_heads(a, Hq, Hkv, kv_of, order);
  for (int r = 0; r < N; ++r) {
    for (int step = 0; step < N; ++step) {
      const int src = ((r - step) % N + N) % N;  // [SP "Algorithmic Mechanics" item 2]
      a.q = (const char*)q + (size_t)r * C * D * 2;
      a.dout = (const char*)dout + (size_t)r * C * D * 2;
      a.k = (const char*)k + (size_t)src * C * D * 2;
      a.v = (const char*)v + (size_t)src * C * D * 2;
      a.qt = pw + L.P.qt + (size_t)r * D * Cp * 2;
      a.dot = pw + L.P.dot + (size_t)r * D * Cp * 2;
      a.kt = pw + L.P.kt + (size_t)src * D * Cp * 2;
      a.lse2 = (const float*)(pw + L.P.lse2) + (size_t)r * Cp;
      a.ndelta = (const float*)(pw + L.P.delta) + (size_t)r * Cp;
      a.dq = dq_acc + (size_t)r * C * D;
      a.dk = dk_acc + (size_t)src * C * D;
      a.dv = dv_acc + (size_t)src * C * D;
      a.qp = pos_of_rank(r);
      a.kp = pos_of_rank(src);
      if ((st = launch_bwd_pair(a, D, s)) != RA_OK) return st;
    }
  }
  if ((e = launch_f32_to_bf16(dq_acc, dq, (int64_t)B * Hq * S * D, s)) != hipSuccess ||
      (e = launch_f32_to_bf16(dk_acc, dk, (int64_t)B * Hkv * S * D, s)) != hipSuccess ||
      (e = launch_f32_to_bf16(dv_acc, dv, (int64_t)B * Hkv * S * D, s)) != hipSuccess)
    return hip_fail(e, "gradient cast launch");
  return RA_OK;
}

// ---------------------------------------------------------------- Ulysses
ra_status ra_ulysses_all_to_all(const void* src, void* dst, int32_t B, int64_t S, int32_t H,
                                int64_t row_bytes, int32_t P, int32_t inverse, void* stream) {
  g_err[0] = 0;
  if (P < 1) return fail(RA_ERR_SHAPE, "P must be >= 1");
  if (B < 0 || S < 0 || H < 1 || row_bytes < 1) return fail(RA_ERR_SHAPE, "bad sizes");
  if (S % P || H % P)
    return fail(RA_ERR_SHAPE, "S=%lld and H=%d must be divisible by P=%d", (long long)S, H, P);
  if (S > INT32_MAX || (S / P) * H > INT32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "S or (S/P)*H beyond 2^31-1");
  if (inverse != 0 && inverse != 1) return fail(RA_ERR_ARG, "inverse must be 0 or 1");
  if (B == 0 || S == 0) return RA_OK;
  if (!src || !dst) return fail(RA_ERR_NULL, "NULL pointer");
  const uintptr_t bytes = (uintptr_t)B * S * H * row_bytes;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RA_ERR_ARG, "src and dst overlap");
  hipError_t e = launch_ulysses_a2a(src, dst, B, S, H, row_bytes, P, inverse,
                                    reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "all-to-all launch");
  return RA_OK;
}

namespace {
// Workspace of the Ulysses simulation: head-sharded [q][k][v][out] in the
// input dtype, then (bf16) V^T [P*B*Hkv/P][D][Spad].
struct UlyssesLayout {
  int64_t Spad;
  size_t q, k, v, o, vt, total;
};
UlyssesLayout ulysses_layout(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                             ra_dtype dt) {
  auto up = [](size_t x) { return (size_t)round_up((int64_t)x, 256); };
  UlyssesLayout L{};
  const size_t es = esize(dt);
  L.Spad = round_up(S, kVtAlign);
  const size_t qb = up((size_t)B * Hq * S * D * es), kb = up((size_t)B * Hkv * S * D * es);
  L.q = 0;
  L.k = qb;
  L.v = qb + kb;
  L.o = qb + 2 * kb;
  L.vt = 2 * qb + 2 * kb;
  L.total = L.vt + (dt == RA_BF16 ? up((size_t)B * Hkv * D * L.Spad * 2) : 0);
  return L;
}
}  // namespace

size_t ra_ulysses_sim_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                      ra_dtype dtype, int32_t P) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1 || P < 1 || S % P) return 0;
  if (dtype != RA_BF16 && dtype != RA_F32) return 0;
  return ulysses_layout(B, Hq, Hkv, S, D, dtype).total;
}

ra_status ra_ulysses_sim_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                             int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                             ra_dtype dtype, int32_t P, int32_t causal, float scale,
                             const int32_t* kv_head_of_q, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_err[0] = 0;
  std::vector<uint8_t> kv_of, order;
  ra_status st = check_common(B, Hq, Hkv, D, dtype, kv_head_of_q, scale, kv_of, order);
  if (st != RA_OK) return st;
  if (causal != 0 && causal != 1) return fail(RA_ERR_ARG, "causal must be 0 or 1");
  if (P < 1) return fail(RA_ERR_SHAPE, "P must be >= 1");
  if (Hq % P || Hkv % P)
    return fail(RA_ERR_SHAPE, "Hq=%d and Hkv=%d must be divisible by P=%d (P <= H_KV)", Hq, Hkv, P);
  const int32_t Hqp = Hq / P, Hkvp = Hkv / P;
  for (int h = 0; h < Hq; ++h)
    if (kv_of[h] / Hkvp != h / Hqp)
      return fail(RA_ERR_SHAPE, "query head %d reads KV head %d, held by another rank", h,
                  (int)kv_of[h]);
  if (S < 0) return fail(RA_ERR_SHAPE, "S must be >= 0");
  if (S % P) return fail(RA_ERR_SHAPE, "S=%lld not divisible by P=%d", (long long)S, P);
  if (S == 0) return RA_OK;
  if (S > INT32_MAX || (S / P) * Hq > INT32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "S or (S/P)*Hq beyond 2^31-1");
  if (!q || !k || !v || !out || !lse) return fail(RA_ERR_NULL, "NULL tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(RA_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  const UlyssesLayout L = ulysses_layout(B, Hq, Hkv, S, D, dtype);
  if (!workspace || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", L.total,
                workspace_bytes);
  if (!aligned(workspace, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t es = esize(dtype);
  char* ws = reinterpret_cast<char*>(workspace);
  char *qh = ws + L.q, *kh = ws + L.k, *vh = ws + L.v, *oh = ws + L.o, *vt = ws + L.vt;
  const bool bf16 = dtype == RA_BF16;
  const int64_t row = (int64_t)D * es;

  // First all-to-all: every rank's q, k, v slices -> head-sharded [P][B][H/P][S][D].
  hipError_t e;
  if ((e = launch_ulysses_a2a(q, qh, B, S, Hq, row, P, 0, s)) != hipSuccess ||
      (e = launch_ulysses_a2a(k, kh, B, S, Hkv, row, P, 0, s)) != hipSuccess ||
      (e = launch_ulysses_a2a(v, vh, B, S, Hkv, row, P, 0, s)) != hipSuccess)
    return hip_fail(e, "all-to-all launch");
  if (bf16 && (e = launch_vt_transpose(vh, vt, (int64_t)B * Hkv, 1, S, L.Spad, D, S * D, s)) !=
                  hipSuccess)
    return hip_fail(e, "V transpose launch");

  // Local attention of each rank: its Hq/P heads over the whole sequence.
  const PosDesc all{1, (int32_t)S, 0, 0, 1};
  const int64_t pairs = pairs_between(all, S, all, S, causal);
  for (int j = 0; j < P; ++j) {
    std::vector<uint8_t> lkv(Hqp), lorder;
    for (int h = 0; h < Hqp; ++h) lkv[h] = (uint8_t)(kv_of[j * Hqp + h] - j * Hkvp);
    lorder.resize(Hqp);
    for (int h = 0; h < Hqp; ++h) lorder[h] = (uint8_t)h;
    std::stable_sort(lorder.begin(), lorder.end(),
                     [&](uint8_t x, uint8_t y) { return lkv[x] < lkv[y]; });
    AttnArgs a;
    memset(&a, 0, sizeof a);
    const size_t qoff = (size_t)j * B * Hqp * S * D, koff = (size_t)j * B * Hkvp * S * D;
    a.q = qh + qoff * es;
    a.q_bs = (int64_t)Hqp * S * D;
    a.q_hs = S * D;
    a.k = kh + koff * es;
    a.k_bs = (int64_t)Hkvp * S * D;
    a.k_hs = S * D;
    if (bf16) {
      a.v = vt + (size_t)j * B * Hkvp * D * L.Spad * 2;
      a.v_bs = (int64_t)Hkvp * D * L.Spad;
      a.v_hs = (int64_t)D * L.Spad;
      a.v_ld = L.Spad;
    } else {
      a.v = vh + koff * es;
      a.v_bs = a.k_bs;
      a.v_hs = a.k_hs;
      a.v_ld = D;
    }
    // accumulate = 0 with a final output: the running state is never read.
    a.fin_out = oh + qoff * es;
    a.fo_bs = a.q_bs;
    a.fo_hs = a.q_hs;
    a.fin_lse = lse + (size_t)j * B * Hqp * S;
    a.fl_bs = (int64_t)Hqp * S;
    a.fl_hs = S;
    a.Cq = (int32_t)S;
    a.Ck = (int32_t)S;
    a.qp = all;
    a.kp = all;
    a.causal = causal;
    a.accumulate = 0;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    fill_attn_work(a, dtype, B, Hqp, S, lkv, lorder);
    const double flops = 4.0 * D * B * Hqp * (double)pairs;
    if ((st = timed_launch(a, dtype, D, s, flops)) != RA_OK) return st;
  }

  // Second all-to-all: head-sharded out -> every rank's sequence slice.
  if ((e = launch_ulysses_a2a(oh, out, B, S, Hq, row, P, 1, s)) != hipSuccess)
    return hip_fail(e, "all-to-all launch");
  return RA_OK;
}

// ---------------------------------------------------------------- USP
namespace {
// Workspace of the USP simulation: head-sharded [q][k][v][out] (input dtype),
// each [P_u][B][H/P_u][S][D] with the ring's rank-major sequence, then one
// ring workspace (reused by the P_u head groups in turn).
struct UspLayout {
  size_t q, k, v, o, ring, ring_bytes, total;
};
UspLayout usp_layout(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D, ra_dtype dt,
                     int32_t P_u, int32_t P_r) {
  auto up = [](size_t x) { return (size_t)round_up((int64_t)x, 256); };
  UspLayout L{};
  const size_t es = esize(dt);
  const size_t qb = up((size_t)B * Hq * S * D * es), kb = up((size_t)B * Hkv * S * D * es);
  L.q = 0;
  L.k = qb;
  L.v = qb + kb;
  L.o = qb + 2 * kb;
  L.ring = 2 * qb + 2 * kb;
  L.ring_bytes = up(ra_ring_sim_workspace_bytes(B, Hq / P_u, Hkv / P_u, S, D, dt, P_r));
  L.total = L.ring + L.ring_bytes;
  return L;
}
}  // namespace

size_t ra_usp_sim_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                  ra_dtype dtype, int32_t P_u, int32_t P_r) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1 || P_u < 1 || P_r < 1) return 0;
  if (Hq % P_u || Hkv % P_u || S % ((int64_t)P_u * P_r)) return 0;
  if (dtype != RA_BF16 && dtype != RA_F32) return 0;
  return usp_layout(B, Hq, Hkv, S, D, dtype, P_u, P_r).total;
}

ra_status ra_usp_sim_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                         int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D, ra_dtype dtype,
                         int32_t P_u, int32_t P_r, ra_layout layout, int32_t causal, float scale,
                         const int32_t* kv_head_of_q, void* workspace, size_t workspace_bytes,
                         void* compute_stream, void* copy_stream) {
  g_err[0] = 0;
  std::vector<uint8_t> kv_of, order;
  ra_status st = check_common(B, Hq, Hkv, D, dtype, kv_head_of_q, scale, kv_of, order);
  if (st != RA_OK) return st;
  if (layout != RA_CONTIGUOUS && layout != RA_ZIGZAG && layout != RA_STRIPED)
    return fail(RA_ERR_ARG, "unknown layout");
  if (causal != 0 && causal != 1) return fail(RA_ERR_ARG, "causal must be 0 or 1");
  if (P_u < 1 || P_r < 1) return fail(RA_ERR_SHAPE, "P_u and P_r must be >= 1");
  if (Hq % P_u || Hkv % P_u)
    return fail(RA_ERR_SHAPE, "Hq=%d and Hkv=%d must be divisible by P_u=%d (P_u <= H_KV)", Hq,
                Hkv, P_u);
  const int32_t Hqp = Hq / P_u, Hkvp = Hkv / P_u;
  for (int h = 0; h < Hq; ++h)
    if (kv_of[h] / Hkvp != h / Hqp)
      return fail(RA_ERR_SHAPE, "query head %d reads KV head %d, held by another device", h,
                  (int)kv_of[h]);
  if (S < 0) return fail(RA_ERR_SHAPE, "S must be >= 0");
  const int64_t P = (int64_t)P_u * P_r;
  if (S % P) return fail(RA_ERR_SHAPE, "S=%lld not divisible by P_u*P_r=%lld", (long long)S,
                         (long long)P);
  if (layout == RA_ZIGZAG && S % (2 * (int64_t)P_r))
    return fail(RA_ERR_SHAPE, "S=%lld not divisible by 2*P_r=%d", (long long)S, 2 * P_r);
  if (S == 0) return RA_OK;
  const int64_t C = S / P_r;  // tokens per node
  if (S > INT32_MAX || (S / P) * Hq > INT32_MAX)
    return fail(RA_ERR_UNSUPPORTED, "S or (S/P)*Hq beyond 2^31-1");
  if (!q || !k || !v || !out || !lse) return fail(RA_ERR_NULL, "NULL tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(RA_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  const UspLayout L = usp_layout(B, Hq, Hkv, S, D, dtype, P_u, P_r);
  if (!workspace || workspace_bytes < L.total)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", L.total,
                workspace_bytes);
  if (!aligned(workspace, 256)) return fail(RA_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t cs = reinterpret_cast<hipStream_t>(compute_stream);
  const size_t es = esize(dtype);
  char* ws = reinterpret_cast<char*>(workspace);
  char *qh = ws + L.q, *kh = ws + L.k, *vh = ws + L.v, *oh = ws + L.o;
  const int64_t row = (int64_t)D * es;
  // device slices of node n: devices n*P_u .. n*P_u + P_u - 1, contiguous
  const size_t node_q = (size_t)P_u * B * (S / P) * Hq * D * es;
  const size_t node_kv = (size_t)P_u * B * (S / P) * Hkv * D * es;

  // Intra-node all-to-all, node by node: the node's tokens land at rows
  // [n*C, (n+1)*C) of every head plane -- rank n of the ring's rank-major order.
  hipError_t e;
  for (int n = 0; n < P_r; ++n) {
    if ((e = launch_ulysses_a2a((const char*)q + n * node_q, qh, B, C, Hq, row, P_u, 0, cs, S,
                                n * C)) != hipSuccess ||
        (e = launch_ulysses_a2a((const char*)k + n * node_kv, kh, B, C, Hkv, row, P_u, 0, cs, S,
                                n * C)) != hipSuccess ||
        (e = launch_ulysses_a2a((const char*)v + n * node_kv, vh, B, C, Hkv, row, P_u, 0, cs, S,
                                n * C)) != hipSuccess)
      return hip_fail(e, "all-to-all launch");
  }
  // The ring across the nodes, once per head group (device u of every node).
  for (int u = 0; u < P_u; ++u) {
    std::vector<int32_t> lmap(Hqp);
    for (int h = 0; h < Hqp; ++h) lmap[h] = kv_of[u * Hqp + h] - u * Hkvp;
    const size_t qo = (size_t)u * B * Hqp * S * D * es, ko = (size_t)u * B * Hkvp * S * D * es;
    st = ra_ring_sim_fwd(qh + qo, kh + ko, vh + ko, oh + qo, lse + (size_t)u * B * Hqp * S, B, Hqp,
                         Hkvp, S, D, dtype, P_r, layout, causal, scale, lmap.data(), ws + L.ring,
                         L.ring_bytes, compute_stream, copy_stream);
    if (st != RA_OK) return st;
  }
  // Reverse all-to-all, node by node.
  for (int n = 0; n < P_r; ++n)
    if ((e = launch_ulysses_a2a(oh, (char*)out + n * node_q, B, C, Hq, row, P_u, 1, cs, S,
                                n * C)) != hipSuccess)
      return hip_fail(e, "all-to-all launch");
  return RA_OK;
}

ra_status ra_device_info(int32_t* compute_units, int32_t* max_clock_khz) {
  g_err[0] = 0;
  if (!compute_units || !max_clock_khz) return fail(RA_ERR_NULL, "NULL output pointer");
  int dev = 0, cus = 0, khz = 0;
  RA_HIP(hipGetDevice(&dev));
  RA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  RA_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev));
  *compute_units = cus;
  *max_clock_khz = khz;
  return RA_OK;
}

ra_status ra_mfma_probe_bf16(int32_t iters, int64_t* out, int64_t out_len, int32_t* waves,
                             void* stream) {
  g_err[0] = 0;
  if (!out || !waves) return fail(RA_ERR_NULL, "NULL pointer");
  if (iters < 1 || iters > (1 << 24)) return fail(RA_ERR_ARG, "iters must be in [1, 2^24]");
  if (!aligned(out, 8)) return fail(RA_ERR_ALIGN, "out must be 8-byte aligned");
  int dev = 0, cus = 0;
  RA_HIP(hipGetDevice(&dev));
  RA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  const int64_t n = (int64_t)cus * (kProbeThreads / 64);
  if (out_len < kProbeWords * n)
    return fail(RA_ERR_WORKSPACE, "out needs %lld entries (got %lld)",
                (long long)(kProbeWords * n), (long long)out_len);
  hipError_t e = launch_mfma_probe(cus, iters, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  *waves = (int32_t)n;
  return RA_OK;
}

ra_status ra_stream_wait(void* stream, int32_t timeout_ms) {
  g_err[0] = 0;
  if (timeout_ms < 0) return fail(RA_ERR_ARG, "timeout_ms must be >= 0 (got %d)", timeout_ms);
  using clock = std::chrono::steady_clock;
  hipEvent_t ev;
  RA_HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  hipError_t e = hipEventRecord(ev, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipEventDestroy(ev);
    return hip_fail(e, "hipEventRecord");
  }
  const clock::time_point t0 = clock::now();
  const clock::duration limit = std::chrono::milliseconds(timeout_ms);
  clock::duration nap = std::chrono::microseconds(20);
  for (;;) {
    e = hipEventQuery(ev);
    if (e != hipErrorNotReady) break;
    const clock::duration waited = clock::now() - t0;
    if (waited >= limit) break;
    std::this_thread::sleep_for(std::min(nap, limit - waited));
    if (nap < std::chrono::milliseconds(1)) nap *= 2;
  }
  // an event destroyed before the stream reaches it is released by the
  // runtime once it completes
  (void)hipEventDestroy(ev);
  if (e == hipSuccess) return RA_OK;
  if (e == hipErrorNotReady)
    return fail(RA_ERR_TIMEOUT, "stream still busy after %d ms", timeout_ms);
  return hip_fail(e, "hipEventQuery");
}

ra_status ra_kernel_timing_enable(int32_t enable) {
  g_err[0] = 0;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.enabled = enable != 0;
  // the events of the first kPreTimed launches exist before any is recorded,
  // so a timed region does not pay for creating them (with no device there is
  // nothing to time: they are created when a launch needs them)
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) ndev = 0;
  while (g_timing.enabled && ndev > 0 && g_timing.ev.size() < 2 * kPreTimed) {
    hipEvent_t e;
    RA_HIP(hipEventCreateWithFlags(&e, kTimingEventFlags));
    g_timing.ev.push_back(e);
  }
  return RA_OK;
}

ra_status ra_kernel_timing_read(double* total_ms, int64_t* launches, double* useful_flops) {
  g_err[0] = 0;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  double ms = 0.0;
  for (size_t i = 0; i < g_timing.used; ++i) {
    RA_HIP(hipEventSynchronize(g_timing.ev[2 * i + 1]));
    float t = 0.f;
    RA_HIP(hipEventElapsedTime(&t, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]));
    ms += t;
  }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = g_timing.launches;
  if (useful_flops) *useful_flops = g_timing.flops;
  g_timing.used = 0;
  g_timing.launches = 0;
  g_timing.flops = 0.0;
  return RA_OK;
}

}  // extern "C"
