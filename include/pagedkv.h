/*
 * pagedkv.h - batched-decode PagedAttention for AMD MI355X (gfx950).
 *
 * C ABI of libpagedkv.so.  Every entry point takes plain pointers and sizes;
 * no allocation, no synchronisation and no state is kept by the library
 * (thread-safe), except for the per-GPU scratch of paged_decode_step_static
 * (see there).  Device pointers are caller-owned HIP device memory; work
 * is enqueued on `stream` (a hipStream_t passed as void*, NULL = the null
 * stream) and the call returns without waiting for it.
 *
 * The method (page titles, sections):
 *  - "Distributed LLM Inference Serving Platform", section 2: a sequence's
 *    KV cache lives in fixed 16-token blocks taken from a pool; a per-
 *    sequence block table maps logical block n (tokens 16n..16n+15) to a
 *    physical block.  Section 5.1: each decode step writes the new token's
 *    K/V into its physical block, then the sequence's single new query
 *    token attends over every block in its table.
 *  - "Roadmap: vLLM-style serving features for TornadoVM batched decode":
 *    B independent sequences advance one token per step (Core batched
 *    decode); block-pool KV with a per-slot block table (Serving /
 *    scheduling); Qwen3's per-head QK-norm + split-half RoPE (Core batched
 *    decode); a quantized FP8 KV cache (Sampling / logits).
 *
 * Layouts (row-major, the pages fix none):
 *   q, out       [B][Hq][D]          fp16
 *   k/v pool     [NB][Hkv][BS][D]    fp16, or E4M3 bytes (OCP FN format)
 *   k/v scale    [NB][Hkv]           fp32, E4M3 only: value = e4m3(code) * scale
 *   block_tables [B][MBS]            int32 physical block ids
 *   context_lens [B]                 int32, valid tokens incl. this step's
 *   slot_mapping [T]                 int64, block * BS + row; < 0 = skip
 *   part_out     [B][Hq][P][D]       fp32 (P = max_partitions)
 *   part_max     [B][Hq][P]          fp32
 *   part_sum     [B][Hq][P]          fp32
 * q head h reads kv head h / (Hq / Hkv) (contiguous GQA groups).
 *
 * Supported shapes: D in {64, 128}; BS == 16, and BS == 32 also for
 * paged_kv_append, paged_kv_append_e4m3, paged_kv_copy_blocks and the
 * balanced paged_decode_step ("Distributed LLM Inference Serving
 * Platform", section 12: 16 or 32 tokens per physical block; the kernels
 * read a 32-token block as two 16-token tiles); Hq % Hkv == 0 with
 * Hq / Hkv in {1, 2, 4, 8}; partition_size 0 or a positive multiple of 16
 * no larger than 16384; MBS * BS <= 2^24.
 *
 * Errors: arguments are checked on the host before anything is enqueued;
 * a failed check returns PKV_EINVAL or PKV_EUNSUPPORTED and enqueues
 * nothing.  A failed launch returns PKV_ELAUNCH.  Device-resident data is
 * the caller's contract and is NOT checked: block ids < NB for the first
 * ceil(L/BS) table entries, 0 <= context_lens[b] <= MBS*BS, distinct slots
 * < NB*BS.  The result never depends on pool bytes outside a sequence's
 * first context_lens[b] rows (they may hold NaN).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,       /* null/misaligned pointer, inconsistent sizes      */
  PKV_EUNSUPPORTED = -2, /* valid but not built: head_dim, group, block size */
  PKV_ELAUNCH = -3,      /* the HIP launch itself failed                     */
  PKV_ENOSPACE = -4      /* paged_decode_step_static: the batch does not fit
                            the library's static scratch                     */
} pkv_status;

typedef enum { PKV_KV_F16 = 0, PKV_KV_E4M3 = 1 } pkv_kv_dtype;

/*
 * PKV_KV_SHARED_BLOCKS - a hint OR-ed into the kv_dtype argument of
 * paged_attn_decode and paged_decode_step: some physical blocks are mapped by
 * several sequences' tables in this call (a prefix shared through reference
 * counts, or the blocks of forked sequences; "Distributed LLM Inference
 * Serving Platform", sections 2 and 11).  Without it every KV tile is read
 * once per call and is loaded with the non-temporal (streaming) cache
 * policy; with it the KV tiles are loaded with the default policy, so that
 * the later readers of a shared block find it in L2 or the Infinity Cache.
 * The results are bitwise the same either way; only speed differs.  Any
 * other bit above the dtype is PKV_EINVAL.
 */
enum { PKV_KV_SHARED_BLOCKS = 0x100 };

/*
 * paged_kv_append - write this step's new K/V rows into their pool slots.
 *
 * "Distributed LLM Inference Serving Platform", section 5.1: K/V of new
 * tokens go straight into the sequence's assigned physical blocks.  For
 * token i with s = slot_mapping[i] >= 0:
 *     k_pool[s / BS][h][s % BS][:] = k_new[i][h][:]   for every kv head h
 * and likewise for v.  Tokens with s < 0 are skipped.
 *
 * Fused Qwen3 prologue ("Roadmap: vLLM-style serving features for TornadoVM
 * batched decode", Core batched decode) when gamma_k != NULL: every q head
 * (q_inout, rewritten in place) and every k head is first normalised,
 *     r = x / sqrt(mean(x^2) + eps) * gamma            (over D, fp32)
 * then rotated by split-half RoPE at pos = context_lens[i] - 1,
 *     a = pos * rope_theta^(-2j/D)                     (angle in fp64)
 *     y_j = r_j cos a - r_{j+D/2} sin a,  y_{j+D/2} = r_{j+D/2} cos a + r_j sin a
 * and rounded once to fp16.  v is copied unchanged.  Without fusion
 * (gamma_k == NULL) q_inout, gamma_q and context_lens are ignored.
 * In the fused call q_inout [T][Hq][D] and context_lens [T] are per token
 * (one token per sequence).
 *
 * k_new, v_new [T][Hkv][D] fp16 (device); k_pool, v_pool [NB][Hkv][BS][D]
 * fp16 (device, written); slot_mapping [T] int64 (device).  All device
 * pointers 16-byte aligned.  T == 0 is a no-op.
 */
int paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                    const int64_t* slot_mapping, int T, int Hkv, int D, int BS,
                    int64_t NB, void* q_inout, int Hq, const float* gamma_q,
                    const float* gamma_k, const int32_t* context_lens, float eps,
                    float rope_theta, void* stream);

/*
 * paged_attn_decode - one query token per sequence attends over its paged
 * KV ("Distributed LLM Inference Serving Platform", sections 2, 3 and 5.1;
 * "Roadmap: vLLM-style serving features for TornadoVM batched decode",
 * Serving / scheduling):
 *     s_t = scale * <q[b][h], K_b[h/g][t]>,  t < L_b = context_lens[b]
 *     out[b][h] = sum_t softmax(s)_t V_b[h/g][t]
 * One online softmax per (sequence, kv head) is shared by the g q heads of
 * the group.  With kv_dtype == PKV_KV_E4M3 the pools hold E4M3 codes and
 * k_scale / v_scale [NB][Hkv] give each (block, kv head) tile's scale.
 * kv_dtype may carry PKV_KV_SHARED_BLOCKS (cache-policy hint, see above).
 *
 * partition_size == 0: single pass; out [B][Hq][D] fp16 is written
 *   (L_b == 0 gives a zero row); the part_* pointers are ignored.
 * partition_size  > 0: each sequence's context is cut into P_b =
 *   ceil(L_b / partition_size) partitions of that many tokens; for each
 *   (b, h, p < P_b) the kernel writes
 *     part_max[b][h][p] = m_p = max_t s_t            (natural-log units)
 *     part_sum[b][h][p] = l_p = sum_t exp(s_t - m_p)
 *     part_out[b][h][p][:] = sum_t exp(s_t - m_p) V_t / l_p
 *   and out is not touched (may be NULL); paged_attn_reduce combines them.
 *   max_partitions >= ceil(MBS * BS / partition_size) is required.
 *
 * scale must be finite and > 0.  B == 0 is a no-op.
 */
int paged_attn_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, const int32_t* context_lens, int B,
                      int Hq, int Hkv, int D, int BS, int MBS, int64_t NB, float scale,
                      int kv_dtype, int partition_size, float* part_out, float* part_max,
                      float* part_sum, int max_partitions, void* stream);

/*
 * paged_attn_reduce - combine split-context partitions into the output.
 * With P_b = ceil(context_lens[b] / partition_size), M = max_{p<P_b} m_p
 * and w_p = l_p exp(m_p - M):
 *     out[b][h][:] = sum_p w_p part_out[b][h][p][:] / sum_p w_p   (fp16, RNE)
 * Only p < P_b is read; L_b == 0 gives a zero row.  The summation order is
 * fixed (p ascending), so results are bitwise reproducible.
 */
int paged_attn_reduce(void* out, const float* part_out, const float* part_max,
                      const float* part_sum, const int32_t* context_lens, int B, int Hq,
                      int D, int partition_size, int max_partitions, void* stream);

/*
 * paged_decode_step - one whole decode step, enqueued on `stream` in one or
 * two launches: the three calls above fused, for the common case where each
 * sequence's new token is its last one ("Distributed LLM Inference Serving
 * Platform", section 5.1: write the new token's K/V into its block, then
 * attend over the block table).
 * For every sequence b with L_b = context_lens[b] >= 1:
 *  1. if k_new != NULL, k_new[b] and v_new[b] ([B][Hkv][D] fp16) become token
 *     L_b - 1: they are written to block block_tables[b][(L_b-1)/BS], row
 *     (L_b-1) % BS, of every kv head (the slot paged_kv_append would be
 *     given).  With gamma_k != NULL the Qwen3 QK-norm + split-half RoPE at
 *     pos = L_b - 1 is first applied to the new k and to q, which is
 *     rewritten in place, exactly as paged_kv_append does;
 *  2. q attends over the sequence's paged KV as in paged_attn_decode;
 *  3. each sequence's context is split into pieces that different
 *     workgroups read in parallel, and the pieces of each (sequence, kv
 *     head) are combined as paged_attn_reduce does, so out [B][Hq][D] fp16
 *     is complete when the step's last launch is.  Balanced split: a
 *     (sequence, kv head) that one workgroup reads whole is written by it
 *     directly; the others are combined by a second launch (their first
 *     piece leaves the piece count in `counters`, which that launch reads
 *     and clears), except with QK-norm, where the last piece to finish
 *     combines them in the same launch (it also writes q' back, which must
 *     wait until every piece has read q).  Fixed partitions: the last
 *     partition to finish combines, in the one launch.
 * partition_size == 0: balanced split.  The library gives every wave the
 *   same number of 16-token tiles of the whole batch (whatever the mix of
 *   context lengths); a sequence is cut into at most max_partitions pieces
 *   (3 <= max_partitions <= 64).  Where the pieces fall depends on the whole
 *   batch, so a sequence's rounding can differ between batches (within the
 *   attention tolerance; the same batch gives the same bits on every call).
 *   Callers that need each sequence's bits independent of the rest of the
 *   batch use fixed partitions.
 * partition_size > 0: fixed partitions of that many tokens as in
 *   paged_attn_decode, at most 64 per sequence
 *   (ceil(MBS * BS / partition_size) <= 64), else PKV_EUNSUPPORTED.
 * part_out / part_max / part_sum: [B][Hq][max_partitions]([D]) fp32 scratch
 *   (contents undefined afterwards).  counters: [B][Hkv * CG] uint32 device
 *   memory (CG = 1 unless n_query > 1 needs column groups, see below), all
 *   zero before the first call; each call leaves them zero again.  Calls
 *   sharing counters, scratch or pools must not run concurrently.
 * window > 0: sliding window ("Roadmap: vLLM-style serving features for
 *   TornadoVM batched decode", Models: Gemma 4's sliding-window layers):
 *   the query attends to positions max(0, L_b - window) .. L_b - 1 only, and
 *   blocks before the window are not read.  Balanced split only
 *   (partition_size == 0, else PKV_EUNSUPPORTED); window == 0 is full
 *   attention, window < 0 is PKV_EINVAL.
 * n_query > 1: several new tokens per sequence ("Roadmap: vLLM-style
 *   serving features for TornadoVM batched decode", Deferred / WIP:
 *   speculative decoding verifies drafted tokens in one forward, chunked
 *   prefill puts several tokens of a sequence in one step).  q and out are
 *   [B][n_query][Hq][D], k_new / v_new [B][n_query][Hkv][D]; L_b counts the
 *   new tokens, which take positions L_b - n_query .. L_b - 1, and new token
 *   j attends to positions 0 .. L_b - n_query + j (causal).  The query
 *   columns of a (sequence, kv head), g = Hq / Hkv heads times n_query
 *   tokens, fill the columns of 16-wide products that share every KV byte
 *   read: up to 16 columns (a power of two) use one product, and the new
 *   rows k_new / v_new may be appended in the same launch; more columns
 *   (a multiple of 16, n_query <= 4096, e.g. a 512-token prefill chunk) are
 *   split into CG = g * n_query / 16 column groups, each of which reads the
 *   sequence's KV once, and the new rows must already be in the pools
 *   (k_new == NULL: paged_kv_append with one slot per new token, with its
 *   QK-norm + RoPE per token position if the model has them).  With
 *   gamma_k != NULL (up to 8 columns, e.g. g = 4 and 2 tokens) each new
 *   token's q and k are normalised and rotated at its own position.
 *   Balanced split only, no window (else PKV_EUNSUPPORTED); part_* then
 *   hold [B][n_query * Hq][max_partitions]([D]).  L_b must be 0 or >=
 *   n_query.
 * prefix_blocks > 0: the first prefix_blocks entries of every table row are
 *   the same physical blocks, a shared prompt prefix ("Roadmap: vLLM-style
 *   serving features for TornadoVM batched decode", Serving / scheduling:
 *   a common prefix prefilled once into blocks all sequences map;
 *   "Distributed LLM Inference Serving Platform", sections 2 and 11:
 *   reference-counted shared blocks).  Each prefix tile is then read once
 *   per group of 16 / (Hq / Hkv) sequences, whose q heads fill the columns
 *   of the same products, instead of once per sequence.  The step then
 *   takes two launches on `stream`: the attention writes every piece's
 *   partial and the piece counts (in `counters`), and a second launch
 *   combines each (sequence, kv head) and clears its counter.  Device-data
 *   contract (not checked): those entries agree across the batch, and every
 *   sequence has L_b == 0 or L_b > prefix_blocks * BS (the prefix holds
 *   past tokens only, so the new row never lands in a shared block); a
 *   sequence with 0 < L_b <= prefix_blocks * BS gets no output.  Balanced
 *   split, n_query == 1, no window, no QK-norm (else PKV_EUNSUPPORTED),
 *   max_partitions >= 6 (a sequence's prefix and own parts take up to
 *   max_partitions / 2 pieces each); prefix_blocks < 0 or > MBS is
 *   PKV_EINVAL.  0 = no shared prefix.
 * kv_dtype PKV_KV_E4M3: k_new != NULL (n_query == 1, no QK-norm, else
 *   PKV_EUNSUPPORTED) appends each sequence's new row at position L_b - 1
 *   with paged_kv_append_e4m3's policy, updating k_scale / v_scale (one more
 *   launch, ahead of the attention); k_new == NULL attends to the pools as
 *   they are.  Either dtype may carry PKV_KV_SHARED_BLOCKS.
 * L_b == 0: zero output row, nothing written to the pools, q untouched.
 * Errors and shape limits as for paged_attn_decode and paged_kv_append.
 */
int paged_decode_step(void* out, void* q, const void* k_new, const void* v_new, void* k_pool,
                      void* v_pool, float* k_scale, float* v_scale,
                      const int32_t* block_tables, const int32_t* context_lens, int B, int Hq,
                      int Hkv, int D, int BS, int MBS, int64_t NB, float scale, int kv_dtype,
                      int partition_size, int window, int n_query, int prefix_blocks,
                      const float* gamma_q,
                      const float* gamma_k, float eps, float rope_theta, float* part_out,
                      float* part_max, float* part_sum, uint32_t* counters, int max_partitions,
                      void* stream);

/*
 * paged_kv_append_e4m3 - write this step's new K/V rows into E4M3 blocks,
 * keeping each (block, kv head) scale valid.
 *
 * The quantized (Q8/FP8) KV cache is a listed item of "Roadmap: vLLM-style
 * serving features for TornadoVM batched decode" (Sampling / logits); the
 * pages fix no policy.  The one implemented keeps a block's scale at the
 * running amax of its rows divided by 448 (the largest E4M3 value).  For
 * token i with p = slot_mapping[i] >= 0, block n = p / BS, row r = p % BS,
 * and for K and V of every kv head h separately, in float32:
 *     a = max_d |new[i][h][d]|;  s_old = r > 0 ? scale[n][h] : 0
 *     if a > 448 * s_old: s_new = a / 448, and rows 0..r-1 of the block are
 *         re-encoded c' = enc((dec(c) * s_old) / s_new)  (skipped if s_old = 0)
 *     else s_new = s_old
 *     row r = enc(new / s_new) (zeros while s_new = 0);  scale[n][h] = s_new
 * enc rounds to the nearest E4M3 value (ties to even) after clamping to
 * +-448; dec is exact.  Rows past r and every other block are untouched.
 *
 * k_new, v_new [T][Hkv][D] fp16; k_pool, v_pool [NB][Hkv][BS][D] E4M3 codes
 * (uint8); k_scale, v_scale [NB][Hkv] fp32; slot_mapping [T] int64; all
 * device memory, pools and rows 16-byte aligned.  T == 0 is a no-op.
 * Device-data contract (not checked): the slots of one call lie in distinct
 * blocks (one wave owns a block's scale while it updates it).
 */
int paged_kv_append_e4m3(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                         float* k_scale, float* v_scale, const int64_t* slot_mapping, int T,
                         int Hkv, int D, int BS, int64_t NB, void* stream);

/*
 * paged_kv_copy_blocks - copy whole physical blocks for copy-on-write.
 *
 * "Distributed LLM Inference Serving Platform", section 11 (worked solution
 * of Lab 1, copy-on-write for parallel sampling) and section 7 (block
 * manager): a sequence that appends into a tail block other sequences still
 * share takes a fresh block and the tokens already written are copied into
 * it.  For every i < n:
 *     k_pool[dst[i]] = k_pool[src[i]],  v_pool[dst[i]] = v_pool[src[i]]
 * (all Hkv heads and BS rows of the block), and with kv_dtype PKV_KV_E4M3
 *     k_scale[dst[i]][:] = k_scale[src[i]][:],  v_scale likewise.
 * Nothing else changes.
 *
 * k_pool, v_pool [NB][Hkv][BS][D] fp16 or E4M3 bytes (device, 16-byte
 * aligned); k_scale, v_scale [NB][Hkv] fp32 (device, E4M3 only, else
 * ignored); src, dst [n] int32 (device).  n == 0 is a no-op.
 * Device-data contract (not checked): 0 <= src[i], dst[i] < NB; the dst[i]
 * are distinct and none of them is also a source (otherwise the result is
 * undefined).  One workgroup per (pair, pool); the copy is HBM bound.
 */
int paged_kv_copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                         const int32_t* src, const int32_t* dst, int n, int Hkv, int D, int BS,
                         int64_t NB, int kv_dtype, void* stream);

/*
 * paged_decode_step_static - paged_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same step, with the split-context
 * partials and arrival counters kept in a scratch array the library holds
 * in each GPU's memory (32 MiB per GPU, taken when the library's code is
 * loaded on that GPU and held until the process ends) instead of a
 * caller-owned workspace.  Arguments are those of paged_decode_step without
 * part_out / part_max / part_sum / counters / max_partitions; the caller
 * still passes every input and output.  Nothing is allocated or freed: no
 * hipMalloc, no allocating library routine.
 *
 * Limits: B * Hkv <= 262144, and the partials of every output row must fit
 * the remaining 31 MiB; the pieces per sequence are
 * paged_decode_step_static_partitions(...) (balanced split: 16, or fewer for
 * large batches, at least 3; fixed partitions: ceil(MBS * BS /
 * partition_size)).  A batch beyond that returns PKV_ENOSPACE and enqueues
 * nothing.  The first call on each GPU also enqueues, on its stream and
 * ahead of its step, one small kernel that zeroes the counters (every step
 * leaves them at zero).
 *
 * Every call on one GPU shares that GPU's scratch: calls that overlap on
 * one GPU (other streams, other host threads) race and give undefined
 * results.  Results equal paged_decode_step's with max_partitions set to
 * paged_decode_step_static_partitions(...).
 */
int paged_decode_step_static(void* out, void* q, const void* k_new, const void* v_new,
                             void* k_pool, void* v_pool, float* k_scale,
                             float* v_scale, const int32_t* block_tables,
                             const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                             int MBS, int64_t NB, float scale, int kv_dtype, int partition_size,
                             int window, int n_query, int prefix_blocks, const float* gamma_q,
                             const float* gamma_k, float eps, float rope_theta, void* stream);

/* Pieces per sequence paged_decode_step_static uses for these sizes (>= 1),
   or PKV_EINVAL / PKV_ENOSPACE.  Host only. */
int paged_decode_step_static_partitions(int B, int Hq, int Hkv, int D, int BS, int MBS,
                                        int n_query, int partition_size);

/* Bytes of part_out + part_max + part_sum for the given sizes (0 on overflow). */
size_t paged_attn_workspace_size(int B, int Hq, int D, int max_partitions);

/* Static description of a pkv_status code. */
const char* pkv_strerror(int status);

/*
 * Host-only argument checks used by the entry points above (no HIP call;
 * safe without a GPU).  Same arguments, same return codes.
 */
int pkv_validate_append(const void* k_new, const void* v_new, const void* k_pool,
                        const void* v_pool, const int64_t* slot_mapping, int T, int Hkv,
                        int D, int BS, int64_t NB, const void* q_inout, int Hq,
                        const float* gamma_q, const float* gamma_k,
                        const int32_t* context_lens, float eps, float rope_theta);
int pkv_validate_decode(const void* out, const void* q, const void* k_pool,
                        const void* v_pool, const float* k_scale, const float* v_scale,
                        const int32_t* block_tables, const int32_t* context_lens, int B,
                        int Hq, int Hkv, int D, int BS, int MBS, int64_t NB, float scale,
                        int kv_dtype, int partition_size, const float* part_out,
                        const float* part_max, const float* part_sum, int max_partitions);
int pkv_validate_step(const void* out, const void* q, const void* k_new, const void* v_new,
                      const void* k_pool, const void* v_pool, const float* k_scale,
                      const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                      int MBS, int64_t NB, float scale, int kv_dtype, int partition_size,
                      int window, int n_query, int prefix_blocks, const float* gamma_q,
                      const float* gamma_k,
                      float eps,
                      float rope_theta, const float* part_out, const float* part_max,
                      const float* part_sum, const uint32_t* counters, int max_partitions);
int pkv_validate_reduce(const void* out, const float* part_out, const float* part_max,
                        const float* part_sum, const int32_t* context_lens, int B, int Hq,
                        int D, int partition_size, int max_partitions);
int pkv_validate_append_e4m3(const void* k_new, const void* v_new, const void* k_pool,
                             const void* v_pool, const float* k_scale, const float* v_scale,
                             const int64_t* slot_mapping, int T, int Hkv, int D, int BS,
                             int64_t NB);
int pkv_validate_copy(const void* k_pool, const void* v_pool, const float* k_scale,
                      const float* v_scale, const int32_t* src, const int32_t* dst, int n,
                      int Hkv, int D, int BS, int64_t NB, int kv_dtype);

/*
 * pkv_stream_read - read a device buffer once, front to back, as fast as the
 * GPU allows.  A measurement yardstick, not part of the attention path: the
 * bench times it to report the step's KV rate as a fraction of the read rate
 * this GPU actually reaches (the spec sheet's 8 TB/s is not reached by any
 * kernel).
 *
 * buf: device memory, 16-byte aligned, bytes a multiple of 16 (0 is a
 * no-op).  sink: one uint32 of device memory; it is written only if the XOR
 * of all 32-bit words read equals 0x9E3779B9 (so that the reads cannot be
 * dropped), and then receives that value.  Returns PKV_EINVAL for a null
 * pointer, misalignment or a bad size, PKV_ELAUNCH if the launch fails.
 */
int pkv_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * pkv_tile_read - read a list of (block, kv head) tiles of a K and a V pool,
 * each once, with the decode step's lane pattern (16 rows of K and of V per
 * tile, as the step loads a 16-token tile for its products), the list cut
 * into `waves` equal contiguous ranges, one single-wave workgroup each, and
 * each XCD's ranges contiguous in the list, as the balanced step splits its
 * tiles.  Nothing is computed with the data.  A measurement yardstick, not
 * part of the attention path: the bench runs it over the tiles a step
 * reads, in the step's order and with its cache policies, and reports the
 * step's KV rate as a fraction of what the GPU delivers for that access
 * pattern (its practical read ceiling, which the streaming read does not
 * give: paged tiles are 4-8 KiB pieces at scattered addresses).
 *
 * k_pool, v_pool: device pools of pool_tiles tiles each; a tile is 16 rows
 *   of row_bytes = 256 (fp16, D = 128), 128 (fp16 D = 64, or E4M3 D = 128)
 *   or 64 (E4M3, D = 64), i.e. tile t of a pool [NB][Hkv][16][D] is
 *   (block t / Hkv, kv head t % Hkv).
 * ids: n int32 on the device; id >= 0 reads tile id with the non-temporal
 *   policy, id < 0 reads tile ~id with the default one (a tile other readers
 *   share); ids past the pools are clamped to the last tile.
 * waves: workgroups, 1 .. 65536 (the step runs 4 per CU for fp16 and 8 for
 *   E4M3).  sink: one uint32 of device memory, written only if the XOR of the
 *   words a lane read equals 0x9E3779B9.
 * Returns PKV_EINVAL for a null pointer, n < 0, pool_tiles < 1, waves out of
 * range or another row_bytes; PKV_ELAUNCH if the launch fails; n == 0 is a
 * no-op.
 */
int pkv_tile_read(const void* k_pool, const void* v_pool, int64_t pool_tiles, const int32_t* ids,
                  int64_t n, int row_bytes, int waves, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
