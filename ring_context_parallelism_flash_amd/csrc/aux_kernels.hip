// Memory-bound helper kernels: the V -> V^T block transpose that feeds the
// bf16 attention kernel, the standalone log-sum-exp merge, the zigzag and
// striped layout permutes and the Ulysses all-to-all.
#include <math.h>

#include "ra_internal.h"

namespace ra {
namespace {

// All-to-all tiles: at most this many bytes per workgroup, heads per table.
constexpr int64_t kA2aTileBytes = 64 * 1024;
constexpr int kA2aMaxHeads = 1024;

// Streaming (non-temporal) 16-byte loads and stores for the copies and the
// merge: no kernel here reads its data twice, and with the non-temporal hint
// a 2 GiB permute moves 6.2-6.3 TB/s instead of 5.7-5.8. Narrower element
// types load and store plainly.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
  if constexpr (sizeof(V) == 16) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    V v;
    __builtin_memcpy(&v, &x, 16);
    return v;
  } else {
    return *p;
  }
}
template <typename V>
__device__ __forceinline__ void stream_store(V* p, const V& v) {
  if constexpr (sizeof(V) == 16) {
    u32x4 x;
    __builtin_memcpy(&x, &v, 16);
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
  } else {
    *p = v;
  }
}

// ---------------------------------------------------------------------------
// V^T blocks. One workgroup transposes a 64-key x D tile through LDS: it reads
// 16-byte chunks along D (coalesced) and writes 16-byte chunks along keys.
// Columns C..Cpad-1 of every block are written as zeros so the attention
// kernel can read whole 64-key tiles without bounds checks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void vt_transpose_kernel(const __bf16* __restrict__ v,
                                                           __bf16* __restrict__ vt, int64_t nblk,
                                                           int64_t C, int64_t Cpad, int64_t v_bh) {
  constexpr int LD = D + 8;  // bf16 elements per LDS row (16-byte pad)
  __shared__ __attribute__((aligned(16))) __bf16 tile[64 * LD];
  const int64_t bh = blockIdx.z, blk = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * 64;  // first column of this tile
  const __bf16* src = v + bh * v_bh + (blk * C) * D;
  __bf16* dst = vt + ((bh * nblk) + blk) * (int64_t)D * Cpad;
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;  // 16-byte chunks per V row
  for (int c = tid; c < 64 * CPR; c += 256) {
    const int row = c / CPR, col = c % CPR;
    const int64_t t = t0 + row;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (t < C) val = *reinterpret_cast<const uint4*>(src + t * D + col * 8);
    *reinterpret_cast<uint4*>(&tile[row * LD + col * 8]) = val;
  }
  __syncthreads();
  // each thread assembles 8 consecutive keys of one d row
  for (int c = tid; c < D * 8; c += 256) {
    const int d = c / 8, kc = c % 8;
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    bf16x8 out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = tile[(kc * 8 + j) * LD + d];
    const int64_t t = t0 + kc * 8;
    if (t < Cpad) *reinterpret_cast<bf16x8*>(dst + (int64_t)d * Cpad + t) = out;
  }
}

// ---------------------------------------------------------------------------
// lse merge: (out, lse) <- merge((out, lse), (out_b, lse_b)). Pass 1 updates
// the output rows reading both lse arrays; pass 2, ordered after it on the
// same stream, rewrites lse. No thread can therefore read a merged lse. The
// output pass moves four consecutive floats per thread on the vector path.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge_weights(float la, float lb, float& ln, float& ca, float& cb) {
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) {
    ln = -INFINITY;
    ca = 0.f;
    cb = 0.f;
    return;
  }
  const float mn = fminf(la, lb);
  ln = mx + log1pf(expf(mn - mx));
  ca = (la == -INFINITY) ? 0.f : expf(la - ln);
  cb = (lb == -INFINITY) ? 0.f : expf(lb - ln);
}

__global__ __launch_bounds__(256) void lse_merge_vec4(float* __restrict__ out,
                                                      const float* __restrict__ lse,
                                                      const float* __restrict__ out_b,
                                                      const float* __restrict__ lse_b,
                                                      int64_t rows, int dq) {
  // dq = D / 4 float4 groups per row
  const int64_t total = rows * dq;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / dq;
    const float la = lse[r], lb = lse_b[r];
    float ln, ca, cb;
    merge_weights(la, lb, ln, ca, cb);
    const float4 a = stream_load(reinterpret_cast<const float4*>(out) + i);
    const float4 b = stream_load(reinterpret_cast<const float4*>(out_b) + i);
    float4 o;
    o.x = fmaf(a.x, ca, b.x * cb);
    o.y = fmaf(a.y, ca, b.y * cb);
    o.z = fmaf(a.z, ca, b.z * cb);
    o.w = fmaf(a.w, ca, b.w * cb);
    stream_store(reinterpret_cast<float4*>(out) + i, o);
  }
}

// One pass: the D/4 threads of a row sit in one wave, read both lse values,
// update the row's float4 groups, and the row's first thread writes the new
// lse. The store is issued after the wave's loads of that lse have returned
// (it depends on them), and no other wave touches the row. dq must divide 64.
__global__ __launch_bounds__(256) void lse_merge_rows(float* __restrict__ out,
                                                      float* __restrict__ lse,
                                                      const float* __restrict__ out_b,
                                                      const float* __restrict__ lse_b,
                                                      int64_t rows, int dq) {
  const int64_t total = rows * dq;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / dq;
    float ln, ca, cb;
    merge_weights(lse[r], lse_b[r], ln, ca, cb);
    const float4 a = stream_load(reinterpret_cast<const float4*>(out) + i);
    const float4 b = stream_load(reinterpret_cast<const float4*>(out_b) + i);
    float4 o;
    o.x = fmaf(a.x, ca, b.x * cb);
    o.y = fmaf(a.y, ca, b.y * cb);
    o.z = fmaf(a.z, ca, b.z * cb);
    o.w = fmaf(a.w, ca, b.w * cb);
    stream_store(reinterpret_cast<float4*>(out) + i, o);
    if (i - r * dq == 0) lse[r] = ln;
  }
}

__global__ __launch_bounds__(256) void lse_merge_scalar(float* __restrict__ out,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ out_b,
                                                        const float* __restrict__ lse_b,
                                                        int64_t rows, int D) {
  const int64_t total = rows * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / D;
    float ln, ca, cb;
    merge_weights(lse[r], lse_b[r], ln, ca, cb);
    out[i] = fmaf(out[i], ca, out_b[i] * cb);
  }
}

__global__ __launch_bounds__(256) void lse_merge_lse_only(float* __restrict__ lse,
                                                          const float* __restrict__ lse_b,
                                                          int64_t rows) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * blockDim.x) {
    float ln, ca, cb;
    merge_weights(lse[r], lse_b[r], ln, ca, cb);
    lse[r] = ln;
  }
}

// ---------------------------------------------------------------------------
// Zigzag permute: 2N chunks of c rows per outer slice. Rank-major chunk pc
// (rank pc/2, half pc%2) holds sequence chunk pc/2 (half 0) or 2N-1-pc/2.
// ---------------------------------------------------------------------------
template <typename V>
__global__ __launch_bounds__(256) void zigzag_permute_kernel(const char* __restrict__ src,
                                                             char* __restrict__ dst, int64_t outer,
                                                             int twoN, int64_t chunk_vecs,
                                                             int inverse) {
  const int64_t nchunks = outer * twoN;
  for (int64_t y = blockIdx.y; y < nchunks; y += gridDim.y) {
    const int64_t o = y / twoN;
    const int pc = (int)(y - o * twoN);
    const int sc = (pc & 1) ? (twoN - 1 - (pc >> 1)) : (pc >> 1);
    const int64_t from = o * twoN + (inverse ? pc : sc);
    const int64_t to = o * twoN + (inverse ? sc : pc);
    const V* s = reinterpret_cast<const V*>(src) + from * chunk_vecs;
    V* d = reinterpret_cast<V*>(dst) + to * chunk_vecs;
    // two streaming loads in flight per thread before the stores
    const int64_t T = (int64_t)gridDim.x * blockDim.x;
    int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; e + T < chunk_vecs; e += 2 * T) {
      const V v0 = stream_load(s + e), v1 = stream_load(s + e + T);
      stream_store(d + e, v0);
      stream_store(d + e + T, v1);
    }
    for (; e < chunk_vecs; e += T) stream_store(d + e, stream_load(s + e));
  }
}

// ---------------------------------------------------------------------------
// Zero fill of a 16-byte-aligned range whose size is a multiple of 16 bytes:
// a plain kernel (not hipMemsetAsync) so the clear is an ordinary kernel node
// when the caller captures the stream into a graph.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, int64_t n16) {
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = z;
}

}  // namespace

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256),
                     0, s, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_vt_transpose(const void* v, void* vt, int64_t BH, int64_t nblk, int64_t C,
                               int64_t Cpad, int D, int64_t v_bh, hipStream_t s) {
  if (BH == 0 || nblk == 0 || Cpad == 0) return hipSuccess;
  const dim3 grid((unsigned)(Cpad / 64), (unsigned)nblk, (unsigned)BH), block(256);
  if (D == 128)
    hipLaunchKernelGGL(vt_transpose_kernel<128>, grid, block, 0, s,
                       reinterpret_cast<const __bf16*>(v), reinterpret_cast<__bf16*>(vt), nblk, C,
                       Cpad, v_bh);
  else
    hipLaunchKernelGGL(vt_transpose_kernel<64>, grid, block, 0, s,
                       reinterpret_cast<const __bf16*>(v), reinterpret_cast<__bf16*>(vt), nblk, C,
                       Cpad, v_bh);
  return hipGetLastError();
}

hipError_t launch_lse_merge(float* out, float* lse, const float* out_b, const float* lse_b,
                            int64_t rows, int D, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const bool vec = (D % 4 == 0) && ((uintptr_t)out % 16 == 0) && ((uintptr_t)out_b % 16 == 0);
  if (vec && D / 4 <= 64 && (64 % (D / 4)) == 0) {
    const int64_t blocks = (rows * (D / 4) + 255) / 256;
    hipLaunchKernelGGL(lse_merge_rows, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(256), 0, s, out, lse, out_b, lse_b, rows, D / 4);
    return hipGetLastError();
  }
  const int64_t work = vec ? rows * (D / 4) : rows * D;
  const int64_t blocks = (work + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  if (vec)
    hipLaunchKernelGGL(lse_merge_vec4, dim3(grid), dim3(256), 0, s, out, lse, out_b, lse_b, rows,
                       D / 4);
  else
    hipLaunchKernelGGL(lse_merge_scalar, dim3(grid), dim3(256), 0, s, out, lse, out_b, lse_b, rows,
                       D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t lblocks = (rows + 255) / 256;
  hipLaunchKernelGGL(lse_merge_lse_only, dim3((unsigned)(lblocks < 65536 ? lblocks : 65536)),
                     dim3(256), 0, s, lse, lse_b, rows);
  return hipGetLastError();
}

// Striped permute [SP "Causal Masking and Load Balancing": token t on rank
// t mod N]: rank-major row p = r*C + i of each [S]-row slab holds sequence row
// i*N + r. Forward gathers (contiguous writes), inverse scatters (contiguous
// reads). A block copies rpb whole rows at a time, one V-sized element per
// thread when a row has at most 256 of them; longer rows are strided.
template <typename V>
__global__ __launch_bounds__(256) void striped_permute_kernel(const char* __restrict__ src,
                                                              char* __restrict__ dst,
                                                              int64_t rows_total, int64_t S, int N,
                                                              int64_t C, int64_t row_vecs, int rpb,
                                                              int inverse) {
  const int t = threadIdx.x;
  const int sub = rpb > 1 ? t / (int)row_vecs : 0;
  const int e0 = rpb > 1 ? t - sub * (int)row_vecs : t;
  if (sub >= rpb) return;  // no barriers below
  for (int64_t g = (int64_t)blockIdx.x * rpb; g < rows_total; g += (int64_t)gridDim.x * rpb) {
    const int64_t row = g + sub;
    if (row >= rows_total) break;
    const int64_t o = row / S, pr = row - o * S;
    const int64_t r = pr / C, i = pr - r * C;
    const int64_t seq = o * S + i * N + r;
    const V* sp = reinterpret_cast<const V*>(src) + (inverse ? row : seq) * row_vecs;
    V* dp = reinterpret_cast<V*>(dst) + (inverse ? seq : row) * row_vecs;
    if (rpb > 1) {
      stream_store(dp + e0, stream_load(sp + e0));
    } else {
      for (int64_t e = e0; e < row_vecs; e += 256) stream_store(dp + e, stream_load(sp + e));
    }
  }
}

hipError_t launch_striped_permute(const void* src, void* dst, int64_t outer, int64_t S,
                                  int64_t row_bytes, int N, int inverse, hipStream_t s) {
  const int64_t rows = outer * S;
  if (rows == 0 || row_bytes == 0) return hipSuccess;
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
  int vb = 16;
  while (vb > 1 && (al % vb)) vb >>= 1;
  const int64_t row_vecs = row_bytes / vb;
  const int rpb = row_vecs <= 256 ? (int)(256 / row_vecs) : 1;
  const int64_t groups = (rows + rpb - 1) / rpb;
  const dim3 grid((unsigned)(groups < 262144 ? groups : 262144));
  const int64_t C = S / N;
  const char* sp = reinterpret_cast<const char*>(src);
  char* dp = reinterpret_cast<char*>(dst);
  switch (vb) {
    case 16:
      hipLaunchKernelGGL(striped_permute_kernel<uint4>, grid, dim3(256), 0, s, sp, dp, rows, S, N,
                         C, row_vecs, rpb, inverse);
      break;
    case 8:
      hipLaunchKernelGGL(striped_permute_kernel<uint2>, grid, dim3(256), 0, s, sp, dp, rows, S, N,
                         C, row_vecs, rpb, inverse);
      break;
    case 4:
      hipLaunchKernelGGL(striped_permute_kernel<uint32_t>, grid, dim3(256), 0, s, sp, dp, rows, S,
                         N, C, row_vecs, rpb, inverse);
      break;
    case 2:
      hipLaunchKernelGGL(striped_permute_kernel<uint16_t>, grid, dim3(256), 0, s, sp, dp, rows, S,
                         N, C, row_vecs, rpb, inverse);
      break;
    default:
      hipLaunchKernelGGL(striped_permute_kernel<uint8_t>, grid, dim3(256), 0, s, sp, dp, rows, S,
                         N, C, row_vecs, rpb, inverse);
      break;
  }
  return hipGetLastError();
}

// Ulysses all-to-all on one GPU [SP "DeepSpeed Ulysses": the first
// all-to-all gathers the sequence and scatters the heads, the second reverses
// it]. The P ranks' sequence slices are [P][B][Sp][H] rows (rank p holds
// positions p*Sp ..); their head slices are [P][B][Hp][S] rows (rank j holds
// heads j*Hp .. over all S positions, each head's rows contiguous; a head's
// plane of S rows starts every hs_stride rows, at row hs_off, so several
// calls can fill one longer sequence). Both directions gather, so the writes
// are contiguous and every read is one whole row. blockIdx.y walks
// destination planes -- (rank, batch, head) forward, (rank, batch) inverse --
// and a block copies rpb consecutive rows of one plane, so the index
// arithmetic inside a plane is 32-bit.
template <typename V>
__global__ __launch_bounds__(256) void ulysses_a2a_kernel(const char* __restrict__ src,
                                                          char* __restrict__ dst, int B, int S,
                                                          int P, int H, int64_t row_vecs, int rpb,
                                                          int inverse, int64_t hs_stride,
                                                          int64_t hs_off) {
  const int Sp = S / P, Hp = H / P;
  const int t = threadIdx.x;
  const int sub = rpb > 1 ? t / (int)row_vecs : 0;
  const int e0 = rpb > 1 ? t - sub * (int)row_vecs : t;
  if (sub >= rpb) return;  // no barriers below
  const int64_t planes = inverse ? (int64_t)P * B : (int64_t)P * B * Hp;
  const int plane_rows = inverse ? Sp * H : S;
  for (int64_t y = blockIdx.y; y < planes; y += gridDim.y) {
    for (int64_t g = (int64_t)blockIdx.x * rpb; g < plane_rows; g += (int64_t)gridDim.x * rpb) {
      const int r = (int)g + sub;
      if (r >= plane_rows) break;
      int64_t from;
      if (!inverse) {  // plane (j, b, hh), row = position r
        const int hh = (int)(y % Hp);
        const int64_t jb = y / Hp;
        const int b = (int)(jb % B), j = (int)(jb / B);
        const int p = r / Sp, i = r - p * Sp;
        from = (((int64_t)p * B + b) * Sp + i) * H + (int64_t)j * Hp + hh;
      } else {  // plane (p, b), row = (i, h)
        const int b = (int)(y % B), p = (int)(y / B);
        const int i = r / H, h = r - i * H;
        const int j = h / Hp, hh = h - j * Hp;
        from = (((int64_t)j * B + b) * Hp + hh) * hs_stride + hs_off + (int64_t)p * Sp + i;
      }
      const int64_t to = inverse ? y * plane_rows + r : y * hs_stride + hs_off + r;
      const V* sp = reinterpret_cast<const V*>(src) + from * row_vecs;
      V* dp = reinterpret_cast<V*>(dst) + to * row_vecs;
      if (rpb > 1) {
        stream_store(dp + e0, stream_load(sp + e0));
      } else {
        for (int64_t e = e0; e < row_vecs; e += 256) stream_store(dp + e, stream_load(sp + e));
      }
    }
  }
}

// Tiled form of the same all-to-all: one workgroup moves T consecutive
// positions i0 .. i0+T-1 of one (rank p, batch b) for all H heads. On the
// position-major side that tile is one contiguous run of T*H rows; on the
// head-major side it is H runs of T consecutive rows, one per head. Reading
// 256-byte rows at a 16 KiB (forward) or whole-plane (inverse) stride, as the
// row-by-row gather does, keeps a DRAM page open for one row; the tile keeps
// both sides in runs. A thread keeps one vector lane of the row (row_vecs
// divides 256) and walks the tile's rows, head-major offsets coming from a
// per-head table in LDS, so the loop has no integer division. T is a power
// of two dividing S/P.
template <typename V>
__global__ __launch_bounds__(256) void ulysses_a2a_tiled(const char* __restrict__ src,
                                                         char* __restrict__ dst, int B, int Sp,
                                                         int Hp, int P, int row_vecs, int log2T,
                                                         int inverse, int64_t hs_stride,
                                                         int64_t hs_off) {
  __shared__ int64_t head_off[kA2aMaxHeads];
  const int H = Hp * P, T = 1 << log2T;
  const int tiles = Sp >> log2T;
  const int64_t pb = blockIdx.x / tiles;  // p * B + b
  const int i0 = (int)(blockIdx.x - pb * tiles) << log2T;
  const int b = (int)(pb % B), p = (int)(pb / B);
  for (int h = threadIdx.x; h < H; h += 256) {
    const int j = h / Hp, hh = h - j * Hp;
    head_off[h] = ((int64_t)j * B * Hp + hh) * hs_stride;
  }
  __syncthreads();
  const int64_t pm0 = (pb * Sp + i0) * H;  // position-major row of (i0, head 0)
  const int64_t hm0 = (int64_t)b * Hp * hs_stride + hs_off + (int64_t)p * Sp + i0;
  const int R = 256 / row_vecs;  // rows per pass of the workgroup
  const int v = threadIdx.x % row_vecs;
  const int rows = H << log2T;
  const V* s = reinterpret_cast<const V*>(src);
  V* d = reinterpret_cast<V*>(dst);
  for (int n0 = threadIdx.x / row_vecs; n0 < rows; n0 += 4 * R) {
    V x[4];
    int64_t to[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = n0 + u * R;  // tile row: head n >> log2T, position i0 + (n & (T-1))
      if (n < rows) {
        const int h = n >> log2T, il = n & (T - 1);
        const int64_t hm = hm0 + head_off[h] + il, pm = pm0 + (int64_t)il * H + h;
        to[u] = (inverse ? pm : hm) * row_vecs + v;
        x[u] = stream_load(s + (inverse ? hm : pm) * row_vecs + v);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (n0 + u * R < rows) stream_store(d + to[u], x[u]);
  }
}

hipError_t launch_ulysses_a2a(const void* src, void* dst, int32_t B, int64_t S, int32_t H,
                              int64_t row_bytes, int32_t P, int inverse, hipStream_t s,
                              int64_t hs_stride, int64_t hs_off) {
  if (hs_stride <= 0) hs_stride = S;
  if (B == 0 || S == 0 || row_bytes == 0) return hipSuccess;
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
  int vb = 16;
  while (vb > 1 && (al % vb)) vb >>= 1;
  const int64_t row_vecs = row_bytes / vb;
  const int64_t Sp = S / P;
  // tiled form: the largest power-of-two T dividing S/P whose tile of T x H
  // rows stays within kA2aTileBytes
  if (256 % row_vecs == 0 && H <= kA2aMaxHeads) {
    int log2T = 0;
    while (Sp % (2LL << log2T) == 0 && (2LL << log2T) * H * row_bytes <= kA2aTileBytes) ++log2T;
    const int64_t blocks = (int64_t)P * B * (Sp >> log2T);
    if (blocks < (1LL << 24)) {  // a grid's x extent stays below 2^32 work-items
      const char* sp = reinterpret_cast<const char*>(src);
      char* dp = reinterpret_cast<char*>(dst);
      const int Hp = H / P, Spi = (int)Sp, rv = (int)row_vecs;
      const dim3 grid((unsigned)blocks);
      switch (vb) {
        case 16:
          hipLaunchKernelGGL(ulysses_a2a_tiled<uint4>, grid, dim3(256), 0, s, sp, dp, B, Spi, Hp,
                             P, rv, log2T, inverse, hs_stride, hs_off);
          break;
        case 8:
          hipLaunchKernelGGL(ulysses_a2a_tiled<uint2>, grid, dim3(256), 0, s, sp, dp, B, Spi, Hp,
                             P, rv, log2T, inverse, hs_stride, hs_off);
          break;
        case 4:
          hipLaunchKernelGGL(ulysses_a2a_tiled<uint32_t>, grid, dim3(256), 0, s, sp, dp, B, Spi,
                             Hp, P, rv, log2T, inverse, hs_stride, hs_off);
          break;
        case 2:
          hipLaunchKernelGGL(ulysses_a2a_tiled<uint16_t>, grid, dim3(256), 0, s, sp, dp, B, Spi,
                             Hp, P, rv, log2T, inverse, hs_stride, hs_off);
          break;
        default:
          hipLaunchKernelGGL(ulysses_a2a_tiled<uint8_t>, grid, dim3(256), 0, s, sp, dp, B, Spi,
                             Hp, P, rv, log2T, inverse, hs_stride, hs_off);
          break;
      }
      return hipGetLastError();
    }
  }
  const int rpb = row_vecs <= 256 ? (int)(256 / row_vecs) : 1;
  const int64_t planes = inverse ? (int64_t)P * B : (int64_t)P * B * (H / P);
  const int64_t plane_rows = inverse ? (S / P) * H : S;
  const int64_t gx = (plane_rows + rpb - 1) / rpb;
  const dim3 grid((unsigned)(gx < 65536 ? gx : 65536), (unsigned)(planes < 65535 ? planes : 65535));
  const char* sp = reinterpret_cast<const char*>(src);
  char* dp = reinterpret_cast<char*>(dst);
  const int Si = (int)S;
  switch (vb) {
    case 16:
      hipLaunchKernelGGL(ulysses_a2a_kernel<uint4>, grid, dim3(256), 0, s, sp, dp, B, Si, P, H,
                         row_vecs, rpb, inverse, hs_stride, hs_off);
      break;
    case 8:
      hipLaunchKernelGGL(ulysses_a2a_kernel<uint2>, grid, dim3(256), 0, s, sp, dp, B, Si, P, H,
                         row_vecs, rpb, inverse, hs_stride, hs_off);
      break;
    case 4:
      hipLaunchKernelGGL(ulysses_a2a_kernel<uint32_t>, grid, dim3(256), 0, s, sp, dp, B, Si, P,
                         H, row_vecs, rpb, inverse, hs_stride, hs_off);
      break;
    case 2:
      hipLaunchKernelGGL(ulysses_a2a_kernel<uint16_t>, grid, dim3(256), 0, s, sp, dp, B, Si, P,
                         H, row_vecs, rpb, inverse, hs_stride, hs_off);
      break;
    default:
      hipLaunchKernelGGL(ulysses_a2a_kernel<uint8_t>, grid, dim3(256), 0, s, sp, dp, B, Si, P,
                         H, row_vecs, rpb, inverse, hs_stride, hs_off);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_zigzag_permute(const void* src, void* dst, int64_t outer, int64_t S,
                                 int64_t row_bytes, int N, int inverse, hipStream_t s) {
  const int twoN = 2 * N;
  const int64_t chunk_bytes = (S / twoN) * row_bytes;
  if (outer == 0 || chunk_bytes == 0) return hipSuccess;
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)chunk_bytes;
  int vb = 16;
  while (vb > 1 && (al % vb)) vb >>= 1;
  const int64_t chunk_vecs = chunk_bytes / vb;
  const int64_t nchunks = outer * twoN;
  const int64_t gx = (chunk_vecs + 511) / 512;  // two vectors per thread
  const dim3 grid((unsigned)(gx < 1024 ? gx : 1024), (unsigned)(nchunks < 65535 ? nchunks : 65535));
  const char* sp = reinterpret_cast<const char*>(src);
  char* dp = reinterpret_cast<char*>(dst);
  switch (vb) {
    case 16:
      hipLaunchKernelGGL(zigzag_permute_kernel<uint4>, grid, dim3(256), 0, s, sp, dp, outer, twoN,
                         chunk_vecs, inverse);
      break;
    case 8:
      hipLaunchKernelGGL(zigzag_permute_kernel<uint2>, grid, dim3(256), 0, s, sp, dp, outer, twoN,
                         chunk_vecs, inverse);
      break;
    case 4:
      hipLaunchKernelGGL(zigzag_permute_kernel<uint32_t>, grid, dim3(256), 0, s, sp, dp, outer,
                         twoN, chunk_vecs, inverse);
      break;
    case 2:
      hipLaunchKernelGGL(zigzag_permute_kernel<uint16_t>, grid, dim3(256), 0, s, sp, dp, outer,
                         twoN, chunk_vecs, inverse);
      break;
    default:
      hipLaunchKernelGGL(zigzag_permute_kernel<uint8_t>, grid, dim3(256), 0, s, sp, dp, outer,
                         twoN, chunk_vecs, inverse);
      break;
  }
  return hipGetLastError();
}

}  // namespace ra
