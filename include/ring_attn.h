/*
 * ring_attn.h -- C ABI of the MI355X (gfx950) ring-attention library.
 *
 * The library computes the per-device step of Ring Attention / Context
 * Parallelism: exact blockwise softmax attention of a resident query chunk
 * against a sequence of key/value blocks, merged with online softmax, with a
 * causal mask taken from each block's GLOBAL sequence positions.
 *
 * Sources (page title, section):
 *   [CP]  "Context Parallelism" (aiwiki.thehackersbrain.dev): "Ring attention",
 *         "The causal imbalance", and the ring_attention code listing with its
 *         flash_block(q, k, v, out, m, lse, source=...) call.
 *   [SP]  "Sequence Parallelism in Large Language Models: How Megatron-SP,
 *         DeepSpeed Ulysses, and RingAttention Distribute Long Contexts"
 *         (llms.blog): "RingAttention and Blockwise Context Parallelism" --
 *         the 4-GPU ring figure, "Algorithmic Mechanics" (online-softmax
 *         equations for m_new, l_new, O_new), "Overlapping Compute and
 *         Communication", "Causal Masking and Load Balancing"; and "DeepSpeed
 *         Ulysses: Head-to-Sequence All-to-All Transposition" and "Unified
 *         Sequence Parallelism (USP / 2D SP)".
 *   [SCP] "Sequence and Context Parallelism" (praveentn.live): "What it does
 *         not change".
 *
 * Conventions shared by every entry point
 *   - Device pointers are HIP device memory owned by the caller. The library
 *     never allocates device memory; scratch space is passed in as
 *     `workspace`.
 *   - Tensors are dense, row-major and contiguous: q and out are
 *     [B, Hq, rows, D]; k and v are [B, Hkv, rows, D]; lse is [B, Hq, rows].
 *   - `stream` arguments are hipStream_t values passed as void*; NULL is the
 *     default stream. Every call only enqueues work and returns; results are
 *     visible after the caller synchronizes the stream.
 *   - All arguments are checked on the host before anything is enqueued, so a
 *     call that returns an error has enqueued nothing. A fault while a kernel
 *     runs surfaces at the caller's next synchronization.
 *   - lse is the natural-log log-sum-exp of the scaled, allowed scores, in
 *     float32. The identity ("no key seen yet") state is out = 0, lse = -inf.
 *   - Entry points are thread-safe with respect to each other: the library
 *     keeps no state between calls apart from the kernel-timing record (its
 *     own lock) and each thread's last error; a ring call creates its own
 *     stream events. Calls that share output or workspace buffers must be
 *     ordered by the caller.
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  RA_ERR_SHAPE = 2,       /* inconsistent sizes, divisibility, head map, pos   */
  RA_ERR_DTYPE = 3,       /* unknown ra_dtype                                  */
  RA_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. D not 64 or 128) */
  RA_ERR_ALIGN = 5,       /* pointer misaligned (16 B for tensors, 4 B lse)    */
  RA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required          */
  RA_ERR_ARG = 7,         /* other invalid value (scale not finite / <= 0)    */
  RA_ERR_HIP = 8,         /* a HIP runtime call failed; see ra_last_error()   */
  RA_ERR_TIMEOUT = 9      /* ra_stream_wait: the stream did not drain in time */
} ra_status;

typedef enum { RA_BF16 = 0, RA_F32 = 1 } ra_dtype;

/* Sequence layouts [SP "Algorithmic Mechanics" item 1; CP "The causal
 * imbalance"; SP "Causal Masking and Load Balancing"]. CONTIGUOUS: rank r
 * holds tokens [r*C, (r+1)*C), C = S/N. ZIGZAG: the sequence is cut into 2N
 * chunks of c = S/(2N); rank r holds chunks r and 2N-1-r, the early chunk
 * first in its memory. STRIPED: token t goes to rank t mod N; rank r holds
 * tokens r, r+N, r+2N, ... in sequence order. */
typedef enum { RA_CONTIGUOUS = 0, RA_ZIGZAG = 1, RA_STRIPED = 2 } ra_layout;

/* Global sequence positions of the rows of one block: row t (0 <= t < rows)
 * sits at position start[t / seg_len] + (t % seg_len) * stride. nseg is 1 or
 * 2 and nseg * seg_len must equal the block's row count; stride >= 1 (0 is
 * read as 1, so a zero-initialised field keeps the unit-stride meaning).
 * With nseg = 2, start[1] > start[0] + (seg_len - 1) * stride (positions
 * increase with t). All positions must be below 2^31. This is the "source"
 * of the pages' flash_block call generalised to any block: a contiguous rank
 * is {1, C, {r*C}, 1}, a zigzag rank is {2, c, {r*c, (2N-1-r)*c}, 1}, a
 * striped rank is {1, C, {r}, N}. A NULL ra_pos means {1, rows, {0}, 1}. */
typedef struct {
  int32_t nseg;
  int64_t seg_len;
  int64_t start[2];
  int64_t stride;
} ra_pos;

/* Human-readable name of a status code (static string). */
const char* ra_status_str(ra_status s);

/* Detail of the last error returned on the calling thread ("" if none). The
 * string stays valid until the thread's next failing call. */
const char* ra_last_error(void);

/* ------------------------------------------------------------------------
 * ra_block_attn_fwd -- one block of ring attention (the pages' flash_block).
 *
 * [CP listing: flash_block(q, k, v, out, m, lse, source=(rank-step)%world);
 *  SP "Algorithmic Mechanics", online-softmax update; SP "Causal Masking":
 *  position i attends to positions j <= i.]
 *
 * For every batch b, query head h (KV head g = kv_head_of_q[h], or
 * h / (Hq/Hkv) when the map is NULL) and query row i of the block, with
 * allowed(i, j) = !causal || kpos(j) <= qpos(i):
 *   s_ij    = scale * <q[b,h,i,:], k[b,g,j,:]>
 *   lse_blk = ln sum_{allowed j} exp(s_ij)
 *   out_blk = sum_{allowed j} exp(s_ij - lse_blk) * v[b,g,j,:]
 * accumulate = 0: (out, lse) := (out_blk, lse_blk); rows with no allowed key
 *   get out = 0, lse = -inf.
 * accumulate = 1: (out, lse) := merge((out, lse), (out_blk, lse_blk)) with
 *   lse' = ln(e^lse + e^lse_blk),
 *   out' = out * e^(lse - lse') + out_blk * e^(lse_blk - lse');
 *   rows with no allowed key are left untouched.
 *
 * q: [B,Hq,Cq,D]; k, v: [B,Hkv,Ck,D], all of `dtype`, 16-byte aligned.
 * out: float32 [B,Hq,Cq,D] (16-byte aligned); lse: float32 [B,Hq,Cq].
 * D must be 64 or 128. scale must be finite and > 0 (pass 1/sqrt(D) for
 * standard attention; the kernels track the exponent reference on unscaled
 * scores, which preserves their order only for a positive scale). workspace: device scratch of at least
 * ra_block_attn_workspace_bytes(...) bytes, 256-byte aligned (may be NULL
 * when that size is 0); it is clobbered. Cq = 0 or Ck = 0 are valid (a block
 * with no keys is the identity for accumulate = 1).
 * ---------------------------------------------------------------------- */
size_t ra_block_attn_workspace_bytes(int32_t B, int32_t Hkv, int64_t Ck, int32_t D,
                                     ra_dtype dtype);

ra_status ra_block_attn_fwd(const void* q, const void* k, const void* v,
                            float* out, float* lse,
                            int32_t B, int32_t Hq, int32_t Hkv,
                            int64_t Cq, int64_t Ck, int32_t D, ra_dtype dtype,
                            const ra_pos* q_pos, const ra_pos* k_pos,
                            const int32_t* kv_head_of_q, int32_t causal, float scale,
                            int32_t accumulate, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * ra_block_attn_fwd_noalloc -- ra_block_attn_fwd for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, semantics and kernels as ra_block_attn_fwd, without
 * `workspace`: the transposed V block (bf16) lives in a 64 MiB array in the
 * library's code object, one per device, looked up once per device and never
 * allocated or freed by the call. Limit: B * Hkv * D * round_up(Ck, 64) * 2
 * bytes must not exceed 64 MiB (e.g. Hkv = 8, D = 128, Ck <= 32768), else
 * RA_ERR_WORKSPACE and nothing is enqueued; fp32 inputs use no scratch.
 * Every call on one device shares that device's array and overwrites it
 * completely before reading it: calls that overlap on one device (other
 * streams, other threads) race and must be ordered by the caller.
 * ---------------------------------------------------------------------- */
ra_status ra_block_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                    float* out, float* lse,
                                    int32_t B, int32_t Hq, int32_t Hkv,
                                    int64_t Cq, int64_t Ck, int32_t D, ra_dtype dtype,
                                    const ra_pos* q_pos, const ra_pos* k_pos,
                                    const int32_t* kv_head_of_q, int32_t causal, float scale,
                                    int32_t accumulate, void* stream);

/* ------------------------------------------------------------------------
 * ra_lse_merge -- fold one normalised partial into a running one, in place.
 *
 * [SP "Algorithmic Mechanics": m_new = max(m_prev, m_block), l_new, O_new.
 *  With lse = m + ln l the three equations become the log-sum-exp form below;
 *  the printed O_new is exact when O_block is the unnormalised block sum, and
 *  this entry point takes the normalised partial out_b together with lse_b.]
 *
 * For each of `rows` rows (r = 0..rows-1):
 *   lse'[r] = ln(e^lse[r] + e^lse_b[r])
 *   out'[r] = out[r] * e^(lse[r]-lse'[r]) + out_b[r] * e^(lse_b[r]-lse'[r])
 * A partial with lse = -inf contributes nothing; two empty partials stay
 * (0, -inf). out, out_b: float32 [rows, D]; lse, lse_b: float32 [rows]. Any
 * D >= 1; 16-byte aligned rows take the vector path.
 * ---------------------------------------------------------------------- */
ra_status ra_lse_merge(float* out, float* lse, const float* out_b, const float* lse_b,
                       int64_t rows, int32_t D, void* stream);

/* ------------------------------------------------------------------------
 * ra_zigzag_permute -- sequence order <-> zigzag rank-major order.
 *
 * [CP "The causal imbalance": split into 2N chunks, rank i holds chunks i and
 *  2N-1-i.]
 *
 * src and dst are [outer, S, row_bytes] byte arrays (row = one token's bytes,
 * e.g. D*2 for a bf16 head row, 4 for an lse entry). With c = S/(2N), the
 * rank-major index p = r*2c + t holds sequence position
 *   chunk(p)*c + (t mod c),  chunk(p) = r if t < c else 2N-1-r.
 * inverse = 0: dst[rank-major p] = src[sequence position of p] (gather).
 * inverse = 1: dst[sequence position of p] = src[rank-major p] (scatter).
 * The copy is bit-exact. S must be divisible by 2N; src and dst must not
 * overlap. Any alignment is accepted; 16-byte aligned chunks are copied with
 * 16-byte accesses.
 * ---------------------------------------------------------------------- */
ra_status ra_zigzag_permute(const void* src, void* dst, int64_t outer, int64_t S,
                            int64_t row_bytes, int32_t N, int32_t inverse, void* stream);

/* ------------------------------------------------------------------------
 * ra_striped_permute -- sequence order <-> striped rank-major order.
 *
 * [SP "Causal Masking and Load Balancing": striped partitioning assigns
 *  token t to rank t mod N.]
 *
 * src and dst are [outer, S, row_bytes] byte arrays as for ra_zigzag_permute.
 * With C = S/N, the rank-major index p = r*C + i holds sequence position
 * i*N + r (rank r's tokens in sequence order).
 * inverse = 0: dst[rank-major p] = src[sequence position of p] (gather).
 * inverse = 1: dst[sequence position of p] = src[rank-major p] (scatter).
 * The copy is bit-exact. S must be divisible by N; src and dst must not
 * overlap. Any alignment is accepted; 16-byte aligned rows are copied with
 * 16-byte accesses.
 * ---------------------------------------------------------------------- */
ra_status ra_striped_permute(const void* src, void* dst, int64_t outer, int64_t S,
                             int64_t row_bytes, int32_t N, int32_t inverse, void* stream);

/* ------------------------------------------------------------------------
 * ra_ring_sim_fwd -- the whole N-rank ring, simulated on one GPU.
 *
 * [CP listing ring_attention(q, k, v, group) and "Ring attention"; SP figure
 *  "Ring Topology (4 GPUs)" and "Algorithmic Mechanics" item 2: at step k
 *  device i holds the KV block of source (i - k) mod N; SP "Overlapping
 *  Compute and Communication": the next block moves while the current one is
 *  computed.]
 *
 * q: [B,Hq,S,D], k, v: [B,Hkv,S,D] of `dtype`; out: [B,Hq,S,D] of `dtype`;
 * lse: float32 [B,Hq,S]. The sequence axis is in RANK-MAJOR order: rank r's
 * C = S/N rows are rows [r*C, (r+1)*C). For RA_CONTIGUOUS that is sequence
 * order; for RA_ZIGZAG (RA_STRIPED) apply ra_zigzag_permute
 * (ra_striped_permute) with inverse=0 to q, k, v before and with inverse=1
 * to out and lse after.
 *
 * For every virtual rank r = 0..N-1 and step k = 0..N-1 the driver attends
 * rank r's queries to the KV block of rank (r - k) mod N, masked by global
 * positions, and merges it into an fp32 running state; the last step writes
 * out (rounded to `dtype`, round-to-nearest-even) and lse. While step k
 * runs on `compute_stream`, the KV block for step k+1 is copied into the
 * other half of a two-slot buffer on `copy_stream`, ordered by events (the
 * copy waits until the slot's previous reader has finished; the compute waits
 * until the copy has landed). A NULL copy_stream runs the copies on
 * compute_stream. The result equals full attention over the sequence.
 *
 * S must be divisible by N (by 2N for RA_ZIGZAG); D must be 64 or 128;
 * workspace: at least ra_ring_sim_workspace_bytes(...) bytes, 256-byte
 * aligned, clobbered.
 * ---------------------------------------------------------------------- */
size_t ra_ring_sim_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                   ra_dtype dtype, int32_t N);

ra_status ra_ring_sim_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                          ra_dtype dtype, int32_t N, ra_layout layout, int32_t causal,
                          float scale, const int32_t* kv_head_of_q,
                          void* workspace, size_t workspace_bytes,
                          void* compute_stream, void* copy_stream);

/* ------------------------------------------------------------------------
 * ra_block_attn_bwd -- gradients of one query block against one KV block.
 *
 * [SCP "What it does not change": the gradients under context parallelism
 *  are those of single-device attention; SP "The Activation Memory Wall":
 *  the attention probabilities are recomputed in the backward pass.]
 *
 * For query head h of batch b, kv head g = map(h), query row i and allowed
 * key row j (the causal rule and positions of ra_block_attn_fwd):
 *   p_ij    = exp(scale*<q_i,k_j> - lse_i)      (lse: the forward's final lse)
 *   delta_i = <dout_i, out_i>                   (out: the forward's output)
 *   ds_ij   = p_ij * (<dout_i, v_j> - delta_i)
 *   dq_i   += scale * sum_j ds_ij k_j
 *   dk_j   += scale * sum_{h, i} ds_ij q_i      (summed over the heads of g)
 *   dv_j   += sum_{h, i} p_ij dout_i
 * q, out, dout: [B,Hq,Cq,D]; k, v: [B,Hkv,Ck,D], bf16 (RA_F32 returns
 * RA_ERR_UNSUPPORTED), 16-byte aligned. lse: float32 [B,Hq,Cq] (-inf marks a
 * row with no key: it contributes nothing). dq: float32 [B,Hq,Cq,D]; dk, dv:
 * float32 [B,Hkv,Ck,D], 16-byte aligned; the gradients are ADDED to them, so
 * the contributions of several key blocks (a ring) accumulate. workspace: at
 * least ra_block_attn_bwd_workspace_bytes(...) bytes, 256-byte aligned,
 * clobbered (transposed copies of q, dout and k, per-row delta and lse).
 * ---------------------------------------------------------------------- */
size_t ra_block_attn_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t Cq,
                                         int64_t Ck, int32_t D, ra_dtype dtype);

ra_status ra_block_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, float* dq, float* dk, float* dv,
                            int32_t B, int32_t Hq, int32_t Hkv, int64_t Cq, int64_t Ck, int32_t D,
                            ra_dtype dtype, const ra_pos* q_pos, const ra_pos* k_pos,
                            const int32_t* kv_head_of_q, int32_t causal, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * ra_ring_sim_bwd -- the backward of the N-rank ring, simulated on one GPU.
 *
 * [SCP "What it does not change"; SP "Algorithmic Mechanics" item 2: at step
 *  k rank i holds the KV block of source (i - k) mod N.]
 *
 * Inputs as for ra_ring_sim_fwd (rank-major sequence order), plus out and lse
 * (that call's results) and dout: [B,Hq,S,D] of `dtype`. Outputs dq
 * [B,Hq,S,D] and dk, dv [B,Hkv,S,D] of `dtype`, rank-major. For every rank r
 * and step k the driver adds the block pair (rank r's queries, the KV block
 * of rank (r - k) mod N) to fp32 accumulators -- dq at rank r, dk and dv at
 * the source block (in a real ring they travel with the block and return to
 * its owner) -- and finally rounds them to `dtype`. The KV blocks are read in
 * place (no copy stream). bf16 only; D 64 or 128; S divisible by N (by 2N for
 * RA_ZIGZAG). workspace: ra_ring_sim_bwd_workspace_bytes(...) bytes, 256-byte
 * aligned, clobbered. The result equals the gradients of full attention.
 * ---------------------------------------------------------------------- */
size_t ra_ring_sim_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                       ra_dtype dtype, int32_t N);

ra_status ra_ring_sim_bwd(const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                          ra_dtype dtype, int32_t N, ra_layout layout, int32_t causal,
                          float scale, const int32_t* kv_head_of_q, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * ra_ulysses_all_to_all -- the Ulysses head<->sequence all-to-all of P ranks,
 * simulated on one GPU as a layout transform.
 *
 * [SP "DeepSpeed Ulysses: Head-to-Sequence All-to-All Transposition": the
 *  layout diagram and Execution Flow items 2 and 4 -- each rank's [B, S/P, H,
 *  D] slice goes to [B, S, H/P, D]: rank j receives every rank's slice of
 *  heads j*H/P .. (j+1)*H/P - 1; the second all-to-all reverses it.]
 *
 * Rows are row_bytes bytes (one token of one head, e.g. D*2 for bf16).
 * Sequence-sharded: [P][B][S/P][H] rows; rank p's slice holds positions
 * p*S/P .. (p+1)*S/P - 1 (its part of the page's [B, S/P, H, D]).
 * Head-sharded: [P][B][H/P][S] rows; rank j's part holds heads j*H/P .. for
 * positions 0..S-1, each head's S rows contiguous (the page's [B, S, H/P, D]
 * with the local head and sequence axes swapped -- the layout the attention
 * kernel reads, so no separate local transpose is needed).
 * inverse = 0: src sequence-sharded -> dst head-sharded (first all-to-all);
 * inverse = 1: src head-sharded -> dst sequence-sharded (second all-to-all).
 * The copy is bit-exact. S and H must be divisible by P; S and (S/P)*H must
 * be below 2^31; src and dst must not overlap. Any alignment is accepted;
 * 16-byte aligned rows are copied with 16-byte accesses.
 * ---------------------------------------------------------------------- */
ra_status ra_ulysses_all_to_all(const void* src, void* dst, int32_t B, int64_t S, int32_t H,
                                int64_t row_bytes, int32_t P, int32_t inverse, void* stream);

/* ------------------------------------------------------------------------
 * ra_ulysses_sim_fwd -- the Ulysses attention of P ranks, simulated on one GPU.
 *
 * [SP "DeepSpeed Ulysses", Execution Flow items 2-4: all-to-all of q, k, v;
 *  local attention on the full sequence for H/P heads; all-to-all of the
 *  output back. "Communication Cost and Constraints": H divisible by P, and
 *  P <= H_KV under GQA. SCP "What it does not change": the result is that of
 *  single-device attention.]
 *
 * q: [P][B][S/P][Hq][D], k, v: [P][B][S/P][Hkv][D] of `dtype` (rank p's
 * slice holds positions p*S/P ..); out: the same layout as q, of `dtype`.
 * lse: float32 [P][B][Hq/P][S] -- it stays on the rank that computed it,
 * head-sharded (rank j, head j*Hq/P + h, position t). Each rank's attention
 * over positions 0..S-1 is one launch of the forward attention kernel with
 * the cast to `dtype` fused into its epilogue. Hq and Hkv must be divisible
 * by P; kv_head_of_q (NULL: h / (Hq/Hkv)) must map every query head to a KV
 * head of the same rank (kv_head_of_q[h] / (Hkv/P) == h / (Hq/P)). D 64 or
 * 128; S divisible by P and below 2^31; scale > 0. workspace: at least
 * ra_ulysses_sim_workspace_bytes(...) bytes, 256-byte aligned, clobbered
 * (head-sharded q, k, v, out and, for bf16, V^T).
 * ---------------------------------------------------------------------- */
size_t ra_ulysses_sim_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                      ra_dtype dtype, int32_t P);

ra_status ra_ulysses_sim_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                             int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                             ra_dtype dtype, int32_t P, int32_t causal, float scale,
                             const int32_t* kv_head_of_q, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * ra_usp_sim_fwd -- unified sequence parallelism on a P_r x P_u device grid,
 * simulated on one GPU.
 *
 * [SP "Unified Sequence Parallelism (USP / 2D SP)": Ulysses all-to-all across
 *  heads inside a node, the ring circulating (K, V) across nodes; SP
 *  "DeepSpeed Ulysses" for the all-to-all; CP listing / SP "Algorithmic
 *  Mechanics" for the ring.]
 *
 * Device d = n*P_u + u is device u of node n. Node n holds the C = S/P_r
 * positions the ring layout gives ring rank n (contiguous, zigzag or
 * striped), in that rank's memory order; device u holds the contiguous piece
 * u of that list, all heads: q [P_r*P_u][B][S/(P_r*P_u)][Hq][D], k, v
 * [..][Hkv][D] of `dtype`; out: the same layout as q, of `dtype`. The call
 * runs, per node, the all-to-all of q, k, v among its P_u devices (device u
 * then holds the node's C positions for heads u*Hq/P_u ..), the ring across
 * the P_r nodes for every head group (as ra_ring_sim_fwd), and the reverse
 * all-to-all of the output. lse: float32 [P_u][B][Hq/P_u][S] -- head group
 * u, sequence axis in ring rank-major order (node 0's positions, then node
 * 1's, ...). Hq and Hkv divisible by P_u, and kv_head_of_q (NULL: h /
 * (Hq/Hkv)) rank-local as for ra_ulysses_sim_fwd; S divisible by P_r*P_u
 * (and by 2*P_r for RA_ZIGZAG). workspace: ra_usp_sim_workspace_bytes(...)
 * bytes, 256-byte aligned, clobbered. copy_stream as for ra_ring_sim_fwd.
 * ---------------------------------------------------------------------- */
size_t ra_usp_sim_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D,
                                  ra_dtype dtype, int32_t P_u, int32_t P_r);

ra_status ra_usp_sim_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                         int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t D, ra_dtype dtype,
                         int32_t P_u, int32_t P_r, ra_layout layout, int32_t causal, float scale,
                         const int32_t* kv_head_of_q, void* workspace, size_t workspace_bytes,
                         void* compute_stream, void* copy_stream);

/* ------------------------------------------------------------------------
 * Kernel timing for measurement (not part of the computation).
 *
 * While enabled, every attention-kernel launch made by ra_block_attn_fwd,
 * ra_ring_sim_fwd, ra_ulysses_sim_fwd, ra_usp_sim_fwd, ra_block_attn_bwd and
 * ra_ring_sim_bwd is bracketed by a
 * pair of HIP events recorded on the stream it is launched on, and the
 * allowed (query, key) pairs it processes are counted on the host.
 * ra_kernel_timing_read waits for the recorded events, returns the summed
 * kernel time in milliseconds, the number of launches and the useful flops
 * (per allowed pair: 4*D for a forward launch; for a backward pair 8*D for
 * the dk/dv kernel and 2*D for the dq kernel, 10*D in all -- the recomputed
 * scores and the four gradient products), and clears the record. Up to
 * 65536 launches are recorded between reads; later ones are
 * not timed (launches still counts them; total_ms then covers only the
 * first 65536). Enabling creates the events of the first 4096 launches
 * (once per process; later ones are created as launches need them).
 * ---------------------------------------------------------------------- */
ra_status ra_kernel_timing_enable(int32_t enable);
ra_status ra_kernel_timing_read(double* total_ms, int64_t* launches, double* useful_flops);

/* ------------------------------------------------------------------------
 * Device figures behind the roofline (measurement, not computation).
 *
 * ra_device_info: the current device's compute-unit count and its maximum
 * shader clock in kHz (hipDeviceGetAttribute), the two factors of the dense
 * bf16 matrix peak CU x clock x flops/CU/clk. Host-only; enqueues nothing.
 *
 * ra_mfma_probe_bf16: launches as many workgroups of 8 waves as there are
 * compute units, one resident per compute unit (two waves per SIMD); each
 * wave issues 4*iters register-fed v_mfma_f32_32x32x16_bf16 (32768 flops
 * each) and writes five int64 to out[5*w ...] (device memory, caller-owned,
 * 8-byte aligned, out_len >= 5 * waves; wave w belongs to workgroup w / 8):
 * the shader-clock counter (s_memtime) at its start and end, the constant
 * 100 MHz reference counter (s_memrealtime) at its start and end, and a
 * liveness word. *waves (host) receives the wave count (8 x compute units).
 * Over a workgroup's span (earliest start to latest end of its waves),
 * flops/CU/clk = 8 * 4 * iters * 32768 / cycles and the shader clock is
 * cycles / (ticks / 100 MHz). iters in [1, 2^24].
 * Errors: RA_ERR_NULL, RA_ERR_ARG, RA_ERR_ALIGN, RA_ERR_WORKSPACE (out too
 * short), RA_ERR_HIP. Asynchronous on `stream`.
 * ---------------------------------------------------------------------- */
ra_status ra_device_info(int32_t* compute_units, int32_t* max_clock_khz);
ra_status ra_mfma_probe_bf16(int32_t iters, int64_t* out, int64_t out_len, int32_t* waves,
                             void* stream);

/* ------------------------------------------------------------------------
 * ra_stream_wait -- wait for a stream with a time limit (host watchdog).
 *
 * [CP "The causal imbalance": the slowest rank sets the pace of every step;
 *  SCP "When it breaks": a ring whose transfers are not hidden degrades into
 *  a chain of N hops.] A ring step cannot finish before the block it waits
 *  for has landed, so a stalled neighbour or copy stalls the step with no
 *  error of its own. This call lets the host bound that wait instead of
 *  blocking in hipStreamSynchronize.
 *
 * Records an event on `stream` (a hipStream_t as void*, NULL = the default
 * stream) behind everything enqueued there so far and polls it from the
 * calling thread, sleeping between polls (20 us, doubling up to 1 ms).
 * Returns RA_OK once the stream has reached the event, RA_ERR_TIMEOUT if it
 * has not after timeout_ms milliseconds (0: poll once; reaching the event
 * takes the device some microseconds even on an idle stream, so a zero limit
 * can report a timeout there), RA_ERR_ARG for a
 * negative timeout_ms (checked before any HIP call), RA_ERR_HIP if the query
 * reports an error (for example a fault of earlier work). On a timeout the
 * enqueued work is neither cancelled nor disturbed: it runs on, and a later
 * call may wait for it again. Host-only apart from the recorded event; no
 * device memory is touched.
 * ---------------------------------------------------------------------- */
ra_status ra_stream_wait(void* stream, int32_t timeout_ms);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
