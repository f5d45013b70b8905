/*
 * hca.h - C ABI of the Heavily Compressed Attention (HCA) layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources: "ERNIE 5.5 Flash Base" release blog, section 2.1,
 * HCA paragraph; Zhidx article, section "1. Latent-Gated Sparse Attention";
 * model card at nlp.com.ai, architecture paragraph):
 *   an HCA layer stores one cached entry per run of 128 tokens and lets every
 *   query attend to all complete entries together with a short window of the
 *   most recent raw (uncompressed) tokens.  The pages do not fix the pooling
 *   function or the window; this library uses
 *     entry j of KV head h:  Kc[j,h] = sum_{i<128} softmax(w_h)_i * K[128j+i, h]
 *                            (Vc likewise, with the same w_h),
 *     keys of query t:       entries j with 128(j+1) <= t+1, then raw
 *                            positions max(0, t-W+1) .. t (no de-duplication),
 *     one softmax over all of them with scale 1/sqrt(head_dim),
 *     query head q reads KV head q / (Hq/Hkv).
 *
 * Conventions for every entry point
 *  - All tensor arguments are DEVICE pointers to caller-owned memory, row
 *    major with head_dim contiguous.  The library never allocates, frees or
 *    synchronises; every call is asynchronous on `stream` (a hipStream_t, or
 *    NULL for the default stream).  It keeps no mutable global state.
 *  - Host-side argument checks run before anything is enqueued; on failure a
 *    non-zero hca_status is returned and nothing is launched.  A launch error
 *    reported by the HIP runtime returns HCA_ERR_HIP.  Faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - The contents of device metadata arrays (monotone cu_* prefix sums,
 *    lengths within the cache capacity) are preconditions, not checked.
 *  - Outputs must not alias inputs.
 *  - dtype HCA_BF16: Q, K, V, Kc, Vc, rings and O are bfloat16; arithmetic is
 *    fp32 accumulation (scores, softmax, pooling) with bf16 MFMA products;
 *    outputs are rounded to nearest even.  dtype HCA_F32: everything fp32.
 *  - Supported shapes: block == 128; window >= 1; num_q_heads a multiple of
 *    num_kv_heads.  HCA_BF16 attention requires head_dim == 512 and
 *    num_q_heads / num_kv_heads == 64 (the shape of the pages' model: 64 query
 *    heads sharing KV, 512-dim heads); HCA_F32 accepts head_dim 1..1024 and any
 *    group size.  hca_compress accepts any head_dim that is a multiple of 64,
 *    up to 1024, in either dtype.
 */
#ifndef HCA_H
#define HCA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define HCA_API __attribute__((visibility("default")))
#else
#define HCA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hca_status {
  HCA_OK = 0,
  HCA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  HCA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes               */
  HCA_ERR_UNSUPPORTED = 3, /* valid, but not a shape/dtype this build handles  */
  HCA_ERR_WORKSPACE = 4,   /* decode workspace missing or too small            */
  HCA_ERR_HIP = 5          /* the HIP runtime rejected a launch                */
} hca_status;

typedef enum hca_dtype { HCA_F32 = 0, HCA_BF16 = 1 } hca_dtype;

typedef struct hca_params {
  int32_t num_q_heads;  /* Hq                                                 */
  int32_t num_kv_heads; /* Hkv, Hq % Hkv == 0                                 */
  int32_t head_dim;     /* d (keys, queries and values share it)              */
  int32_t block;        /* tokens per compressed entry; must be 128           */
  int32_t window;       /* W >= 1: raw positions max(0,t-W+1)..t are visible  */
  float softmax_scale;  /* <= 0 selects 1/sqrt(head_dim)                      */
  int32_t dtype;        /* hca_dtype of every tensor except w (always fp32)   */
} hca_params;

/*
 * hca_compress - pool every complete 128-token block of K (and V) into one
 * cached entry (release blog, section 2.1, HCA paragraph: one cached entry
 * per 128 tokens).
 *
 *   batch           number of packed sequences B >= 0
 *   total_blocks    host copy of cu_blocks[B] (number of entries written)
 *   cu_seqlens      device int32 [B+1], token offsets of each sequence
 *   cu_blocks       device int32 [B+1], cu_blocks[b+1]-cu_blocks[b] ==
 *                   floor((cu_seqlens[b+1]-cu_seqlens[b]) / 128)
 *   k, v            device [N_tok, Hkv, d] raw keys / values; v may be NULL
 *   w               device fp32 [Hkv, 128] pooling logits
 *   kc, vc          device [total_blocks, Hkv, d] outputs; vc NULL iff v NULL
 *                   (with total_blocks == 0 nothing is read or written and
 *                   every pointer may be NULL)
 *
 * Entry cu_blocks[b]+j, head h = sum_i softmax(w_h)_i * x[cu_seqlens[b]+128j+i, h]
 * accumulated in fp32.  A trailing partial block is not pooled.
 */
HCA_API hca_status hca_compress(const hca_params* params, int32_t batch, int32_t total_blocks,
                        const int32_t* cu_seqlens, const int32_t* cu_blocks,
                        const void* k, const void* v, const float* w,
                        void* kc, void* vc, void* stream);

/*
 * hca_attend_prefill - causal HCA attention for every token of a packed
 * batch (release blog, section 2.1; Zhidx article, section 1: attention over
 * the compressed entries plus a short raw window).
 *
 *   batch, max_seqlen  host: B and max_b (cu_seqlens[b+1]-cu_seqlens[b])
 *   cu_seqlens, cu_blocks  device int32 [B+1] as for hca_compress
 *   q               device [N_tok, Hq, d]
 *   k, v            device [N_tok, Hkv, d] raw keys / values of the batch
 *   kc, vc          device [cu_blocks[B], Hkv, d] entries (from hca_compress)
 *   o               device [N_tok, Hq, d] output
 *
 * Token t (0-based within its sequence) attends to entries 0 ..
 * floor((t+1)/128)-1 of its sequence and to raw tokens max(0,t-W+1) .. t.
 */
HCA_API hca_status hca_attend_prefill(const hca_params* params, int32_t batch, int32_t max_seqlen,
                              const int32_t* cu_seqlens, const int32_t* cu_blocks,
                              const void* q, const void* k, const void* v,
                              const void* kc, const void* vc, void* o, void* stream);

/*
 * hca_attend_prefill_gated_vha - hca_attend_prefill with the attention
 * epilogue fused into the output stage (release blog, section 2.1, last
 * paragraph: a low-rank gated attention output gate and Virtual Head
 * Attention, a cross-head low-rank mixing with identity skip applied after
 * attention and fused into the attention kernel at inference).  With O the
 * attention output of one token and the G = Hq / Hkv heads of one KV head:
 *
 *   y[h] = sigmoid(gate[t, h]) * (O[h] + sum_r U[h, r] sum_h' V[h', r] O[h'])
 *
 *   gate            device fp32 [N_tok, Hq] gate logits (the gate projection
 *                   of the query latent runs upstream), or NULL: no gate
 *   vha_u, vha_v    device fp32 [Hkv, G, vha_rank] mixing factors, both or
 *                   neither NULL; 1 <= vha_rank <= 32
 *
 * The pages fix neither the rank nor the gate granularity: one gate logit
 * per (token, head), mixing within a KV head's group, mixing before the gate.
 * HCA_BF16 only (HCA_ERR_UNSUPPORTED for HCA_F32 with an epilogue); with no
 * gate and no mixing it is hca_attend_prefill.
 */
HCA_API hca_status hca_attend_prefill_gated_vha(const hca_params* params, int32_t batch,
                                        int32_t max_seqlen, const int32_t* cu_seqlens,
                                        const int32_t* cu_blocks, const void* q, const void* k,
                                        const void* v, const void* kc, const void* vc,
                                        const float* gate, const float* vha_u,
                                        const float* vha_v, int32_t vha_rank, void* o,
                                        void* stream);

/*
 * hca_decode_workspace_bytes - size in bytes of the scratch buffer that
 * hca_attend_decode needs for `batch` sequences whose longest cache holds
 * `max_blocks` entries.  Returns 0 for invalid params.
 */
HCA_API size_t hca_decode_workspace_bytes(const hca_params* params, int32_t batch, int32_t max_blocks);

/*
 * hca_attend_decode - one new query per sequence against its HCA cache
 * (release blog, section 2.1: every query sees all complete entries plus the
 * recent raw window).
 *
 *   batch, max_blocks  host: B and max_b floor(L_b / 128)
 *   seqlens         device int32 [B], L_b >= 1 counts the new token, whose
 *                   query sits at position L_b - 1
 *   cu_blocks       device int32 [B+1]; sequence b owns entries
 *                   [cu_blocks[b], cu_blocks[b+1]) and at least floor(L_b/128)
 *   q               device [B, Hq, d]
 *   kc, vc          device [cu_blocks[B], Hkv, d]
 *   kw, vw          device [B, ring_cap, Hkv, d] raw rings: position s of
 *                   sequence b is in slot s % ring_cap; ring_cap >= window
 *   o               device [B, Hq, d] output
 *   workspace       device scratch of workspace_bytes >=
 *                   hca_decode_workspace_bytes(...), 256-byte aligned, any
 *                   contents (it holds per-split partial results between the
 *                   two kernels of one call).  Calls that share one workspace
 *                   must not overlap in time.  HCA_F32 needs no workspace
 *                   (size 0; NULL is accepted).
 */
HCA_API hca_status hca_attend_decode(const hca_params* params, int32_t batch, int32_t max_blocks,
                             const int32_t* seqlens, const int32_t* cu_blocks,
                             const void* q, const void* kc, const void* vc,
                             const void* kw, const void* vw, int32_t ring_cap,
                             void* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * hca_attend_decode_noalloc - hca_attend_decode (bf16 or fp32, no epilogue)
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It takes
 * no workspace: the split partials go to a static device array of
 * HCA_DECODE_NOALLOC_SCRATCH_BYTES (32 MiB) that each GPU the library runs
 * on holds until the process ends, and the call allocates and frees
 * nothing.  Its device address is looked up once per device, on the first
 * call with that device current.
 *
 * Arguments, layouts and results are those of hca_attend_decode (same
 * kernels, bit-identical output).  Errors: as hca_attend_decode, plus
 * HCA_ERR_WORKSPACE when the call needs more scratch than the array holds
 * (hca_decode_workspace_bytes(params, batch, max_blocks) >
 * HCA_DECODE_NOALLOC_SCRATCH_BYTES; 64 sequences at 131072 tokens need
 * 16.9 MB) and HCA_ERR_HIP if the runtime cannot give the array's address.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, or two host threads) race on it; calls on one
 * stream are ordered and safe.
 */
#define HCA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
HCA_API hca_status hca_attend_decode_noalloc(const hca_params* params, int32_t batch, int32_t max_blocks,
                                             const int32_t* seqlens, const int32_t* cu_blocks, const void* q,
                                             const void* kc, const void* vc, const void* kw, const void* vw,
                                             int32_t ring_cap, void* o, void* stream);

/*
 * Serving with a cache: chunks of new tokens and decode steps.
 *
 * A sequence's HCA cache is its compressed entries (one per complete block,
 * release blog, section 2.1) plus a raw ring [B, ring_cap, Hkv, d] holding
 * position s in slot s % ring_cap (the recent raw tokens the window needs).
 * New rows of sequence b are n_b = cu_seqlens[b+1] - cu_seqlens[b] tokens at
 * positions pos0[b] .. pos0[b] + n_b - 1, packed in k / v [N, Hkv, d].
 *
 *   a chunk:        hca_compress_chunk, hca_attend_prefill_chunk, hca_ring_append
 *   a decode step:  hca_compress_chunk and hca_ring_append with one row per
 *                   sequence, then hca_attend_decode
 *
 * The ring must hold positions pos0[b] - ring_cap .. pos0[b] - 1 (those >= 0)
 * when a call starts; hca_ring_append writes the new rows last, since the
 * other two calls read the older rows the new ones replace.  The output of a
 * chunk equals rows pos0[b] .. pos0[b] + n_b - 1 of hca_attend_prefill over
 * the whole sequence.
 */

/*
 * hca_compress_chunk - pool every block the new rows complete: block j with
 * pos0[b] <= 128j + 127 <= pos0[b] + n_b - 1 becomes entry cu_blocks[b] + j
 * (same arithmetic as hca_compress).  Rows of the block before pos0[b] are
 * read from the ring, so ring_cap >= 128.
 *
 *   batch, max_rows  host: B and max_b n_b
 *   cu_seqlens       device int32 [B+1], offsets of the new rows
 *   pos0             device int32 [B], position of each sequence's first new row
 *   cu_blocks        device int32 [B+1], cache layout: sequence b owns entries
 *                    [cu_blocks[b], cu_blocks[b+1]), at least floor((pos0[b] + n_b)/128)
 *   k, v             device [N, Hkv, d] new rows; v may be NULL (then vw, vc too)
 *   w                device fp32 [Hkv, 128] pooling logits
 *   kw, vw           device rings [B, ring_cap, Hkv, d] (read only)
 *   kc, vc           device caches; only the completed entries are written
 *                    (never an index past cu_blocks[b+1])
 */
HCA_API hca_status hca_compress_chunk(const hca_params* params, int32_t batch, int32_t max_rows,
                              const int32_t* cu_seqlens, const int32_t* pos0,
                              const int32_t* cu_blocks, const void* k, const void* v,
                              const float* w, const void* kw, const void* vw, int32_t ring_cap,
                              void* kc, void* vc, void* stream);

/*
 * hca_ring_append - write the last min(n_b, ring_cap) new rows of every
 * sequence into its ring (position s -> slot s % ring_cap); other slots are
 * left as they are.  Pure data movement, bit-exact.
 *
 *   k, v      device [N, Hkv, d] new rows; v may be NULL (then vw too)
 *   kw, vw    device rings [B, ring_cap, Hkv, d], written
 */
HCA_API hca_status hca_ring_append(const hca_params* params, int32_t batch, int32_t max_rows,
                           const int32_t* cu_seqlens, const int32_t* pos0,
                           const void* k, const void* v, void* kw, void* vw,
                           int32_t ring_cap, void* stream);

/*
 * hca_prefill_chunk_workspace_bytes - scratch size for hca_attend_prefill_chunk
 * with `batch` sequences and `total_rows` = cu_seqlens[B] new rows: the
 * window - 1 ring rows before each chunk and the chunk's rows, staged as one
 * run per sequence (K and V).  Returns 0 for invalid params.
 */
HCA_API size_t hca_prefill_chunk_workspace_bytes(const hca_params* params, int32_t batch,
                                         int32_t total_rows);

/*
 * hca_attend_prefill_chunk - HCA attention for the new rows of every
 * sequence (queries at positions pos0[b] ..), over its cache: entries 0 ..
 * floor((t+1)/128) - 1 (the ones completed inside the chunk must already be
 * pooled by hca_compress_chunk) and raw tokens max(0, t-W+1) .. t, from the
 * ring before pos0[b] and from k / v after.
 *
 *   batch, max_seqlen, total_rows  host: B, max_b n_b, cu_seqlens[B]
 *   q               device [N, Hq, d]; o device [N, Hq, d] output
 *   k, v            device [N, Hkv, d] new rows
 *   kc, vc          device caches as for hca_compress_chunk
 *   kw, vw          device rings, ring_cap >= window (read only)
 *   workspace       device scratch of >= hca_prefill_chunk_workspace_bytes,
 *                   256-byte aligned, any contents
 */
HCA_API hca_status hca_attend_prefill_chunk(const hca_params* params, int32_t batch,
                                    int32_t max_seqlen, int32_t total_rows,
                                    const int32_t* cu_seqlens, const int32_t* pos0,
                                    const int32_t* cu_blocks, const void* q, const void* k,
                                    const void* v, const void* kc, const void* vc,
                                    const void* kw, const void* vw, int32_t ring_cap, void* o,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * hca_attend_decode_gated_vha, hca_attend_prefill_chunk_gated_vha - the
 * decode and chunk calls with the attention epilogue of
 * hca_attend_prefill_gated_vha (same arguments and meaning; gate logits are
 * [B, Hq] for decode and [N, Hq] for a chunk).  Decode applies it in the
 * merge of the split partials (fp32 mixing), chunks in the prefill kernel.
 * HCA_BF16 only.
 */
HCA_API hca_status hca_attend_decode_gated_vha(const hca_params* params, int32_t batch,
                                       int32_t max_blocks, const int32_t* seqlens,
                                       const int32_t* cu_blocks, const void* q, const void* kc,
                                       const void* vc, const void* kw, const void* vw,
                                       int32_t ring_cap, const float* gate, const float* vha_u,
                                       const float* vha_v, int32_t vha_rank, void* o,
                                       void* workspace, size_t workspace_bytes, void* stream);
HCA_API hca_status hca_attend_prefill_chunk_gated_vha(
    const hca_params* params, int32_t batch, int32_t max_seqlen, int32_t total_rows,
    const int32_t* cu_seqlens, const int32_t* pos0, const int32_t* cu_blocks, const void* q,
    const void* k, const void* v, const void* kc, const void* vc, const void* kw, const void* vw,
    int32_t ring_cap, const float* gate, const float* vha_u, const float* vha_v, int32_t vha_rank,
    void* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training: the gradient of hca_attend_prefill.  The pages train the model at
 * long context (release blog "ERNIE 5.5 Flash Base", section 2.1; the model
 * card gives the 128K training context) and print no backward: these calls
 * compute the exact derivative of the forward above, HCA_BF16 with 512-dim
 * heads and 64 query heads per KV head only (HCA_ERR_UNSUPPORTED otherwise).
 *
 * hca_attend_prefill_lse - hca_attend_prefill that also writes, per query row,
 * the log-sum-exp of its scaled scores over its visible keys:
 *
 *   lse             device fp32 [N_tok, Hq], natural log,
 *                   lse[t, h] = log sum_j exp(scale q[t,h] . key_j)
 *
 * Same other arguments, errors and ownership as hca_attend_prefill.
 */
HCA_API hca_status hca_attend_prefill_lse(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                          const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                          const void* q, const void* k, const void* v,
                                          const void* kc, const void* vc, void* o, float* lse,
                                          void* stream);

/*
 * hca_attend_prefill_backward_workspace_bytes - scratch bytes that
 * hca_attend_prefill_backward needs (0 for invalid or unsupported params):
 * 4 N_tok Hq (dO . O per row) + 8 N_tok Hkv d (fp32 raw-row gradients)
 * + 8 B Hkv ceil(max_blocks / 32) S 32 d (fp32 partials of the compressed
 * entries, S <= 256 runs of max(64, ceil(max_seqlen / 256)) positions,
 * max_blocks = floor(max_seqlen / 128)) + 512 total_blocks Hkv, each part
 * rounded up to 256 bytes.
 */
HCA_API size_t hca_attend_prefill_backward_workspace_bytes(const hca_params* params, int32_t batch,
                                                           int32_t total_tokens, int32_t total_blocks,
                                                           int32_t max_seqlen);

/*
 * hca_attend_prefill_backward - gradients of a loss L through
 * hca_compress (K and V pooled with softmax(w)) followed by
 * hca_attend_prefill, given dL/dO:
 *
 *   batch, max_seqlen, cu_seqlens, cu_blocks   as for hca_attend_prefill
 *   total_tokens    host: N_tok = cu_seqlens[B]
 *   total_blocks    host: cu_blocks[B]
 *   q, k, v         device bf16 inputs of the forward
 *   w               device fp32 [Hkv, 128] pooling logits
 *   kc, vc          device bf16 [total_blocks, Hkv, d] the forward's entries
 *   o, lse          device: the forward's output and hca_attend_prefill_lse's
 *                   lse
 *   dout            device bf16 [N_tok, Hq, d] dL/dO
 *   dq              device bf16 [N_tok, Hq, d] dL/dq (written)
 *   dk, dv          device bf16 [N_tok, Hkv, d] dL/dk, dL/dv through both the
 *                   raw window and the pooled entries (written)
 *   dw              device fp32 [Hkv, 128] dL/dw (written; zero without a
 *                   complete block)
 *   workspace       device scratch of at least
 *                   hca_attend_prefill_backward_workspace_bytes bytes
 *                   (HCA_ERR_WORKSPACE when NULL or smaller)
 *
 * Per query row and visible key j: P_j = exp(scale q.k_j - lse),
 * dS_j = P_j (dO.v_j - dO.O); dq = scale sum dS_j k_j, a key gets
 * scale dS_j q and its value P_j dO; an entry's gradients reach its block's
 * rows weighted by softmax(w), and dw = p (g - sum p g) with
 * g_i = sum over entries of (dKc . K_i + dVc . V_i).  Deterministic (no
 * atomics).  Outputs must not alias inputs or the workspace.
 */
HCA_API hca_status hca_attend_prefill_backward(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                               int32_t total_tokens, int32_t total_blocks,
                                               const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                               const void* q, const void* k, const void* v, const float* w,
                                               const void* kc, const void* vc, const void* o,
                                               const float* lse, const void* dout, void* dq, void* dk,
                                               void* dv, float* dw, void* workspace, size_t workspace_bytes,
                                               void* stream);

/*
 * Sparse attention of the full-context (MLA) layers, decode step.  The pages
 * (release blog "ERNIE 5.5 Flash Base", section 2.1; Zhidx article, section
 * 1; model card) describe it in outline only: a lightweight indexer scores
 * the past positions of each query, core attention runs over the top-k
 * highest-scoring positions, and these layers use 256-dim heads.  Fixed here
 * (the pages give no indexer form and no k):
 *
 *   score(s) = qi . ki[s]   one int8 indexer head of width 128, exact integer
 *   selection               the topk highest scores among positions 0 .. L-1
 *                           (the query sits at L-1), equal scores to the
 *                           smaller position; all positions when L <= topk
 *   attention               64 query heads of width 256 attend under one
 *                           softmax to the shared key / value rows (one KV
 *                           head, width 256) of the selected positions
 *
 * hca_dsa_decode_workspace_bytes - scratch bytes hca_dsa_decode needs (0 for
 * invalid sizes).
 */
HCA_API size_t hca_dsa_decode_workspace_bytes(int32_t batch, int32_t max_seqlen, int32_t topk);

/*
 * hca_dsa_decode - one query per sequence.
 *
 *   batch, max_seqlen, topk  host: B, max_b L_b (L_b >= 1), k >= 1
 *   softmax_scale   <= 0: 1/16 (1/sqrt(256))
 *   seqlens         device int32 [B]: L_b
 *   cu_rows         device int32 [B]: first cache row of sequence b; its rows
 *                   cu_rows[b] .. cu_rows[b] + L_b - 1 hold positions 0 .. L_b-1
 *   q               device bf16 [B, 64, 256] queries
 *   qi              device int8 [B, 128] indexer queries
 *   k, v            device bf16 [rows, 256] key / value cache
 *   ki              device int8 [rows, 128] indexer keys
 *   o               device bf16 [B, 64, 256] output (written)
 *   sel             device int32 [B, topk] selected positions in increasing
 *                   order, -1 after the first min(topk, L_b) (written)
 *   workspace       device scratch of hca_dsa_decode_workspace_bytes bytes
 *                   (HCA_ERR_WORKSPACE when NULL or smaller)
 *
 * The selection is exact (integer scores), so it is the same on every device.
 * Outputs must not alias inputs.
 */
HCA_API hca_status hca_dsa_decode(int32_t batch, int32_t max_seqlen, int32_t topk, float softmax_scale,
                                  const int32_t* seqlens, const int32_t* cu_rows, const void* q,
                                  const int8_t* qi, const void* k, const void* v, const int8_t* ki, void* o,
                                  int32_t* sel, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement probes.  Not part of the layer: they measure what the part
 * reaches on plain streams of work, so that the benchmark can state the
 * hot-path kernels' fractions against measured ceilings next to the
 * published ones.  All are asynchronous on `stream`; `sink` is a
 * caller-owned device buffer the kernels write so that their work is kept.
 *
 * hca_probe_stream_read - reads every byte of `buf` (device, `bytes` a
 *   multiple of 16) once with 16-byte non-temporal loads; `grid` workgroups
 *   of 256 threads; sink: device uint32 [4 * grid].
 * hca_probe_stream_lds - reads the first floor(bytes / 49152) 48 KiB tiles of
 *   `buf` once through LDS with direct buffer->LDS loads (the attention
 *   kernels' key-tile path), two tiles in flight per workgroup of 256
 *   threads (144 KiB of LDS, so one workgroup per CU); `grid` workgroups;
 *   sink: device uint32 [4 * grid]; bytes < 49152 is HCA_ERR_SHAPE.
 * hca_probe_mfma_bf16 - each of `grid` workgroups (4 wavefronts) runs
 *   `iters` x 4 independent v_mfma_f32_32x32x16_bf16 per wavefront
 *   (32768 flops each); sink: device float [4 + 4 * grid].  sink[0] and
 *   sink[1] receive the shader-clock cycles and the fixed-rate (100 MHz)
 *   ticks that the first wavefront's loop took, whose ratio is the clock the
 *   loop ran at.
 * hca_probe_lds_read - each wavefront of `grid` workgroups reads LDS `iters`
 *   x 8 times: mode 0 one 1 KiB row per instruction (16-byte reads), mode 1
 *   the transposed 8-byte reads of V^T fragments (512 bytes per
 *   instruction); sink: device uint32 [4 * grid].
 * Return HCA_ERR_NULL for a NULL buffer, HCA_ERR_SHAPE for sizes out of
 * range (grid 1 .. 65536, iters >= 1), HCA_ERR_HIP if the launch fails.
 */
HCA_API hca_status hca_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, void* stream);
HCA_API hca_status hca_probe_stream_lds(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, void* stream);
HCA_API hca_status hca_probe_mfma_bf16(int32_t iters, int32_t grid, float* sink, void* stream);
HCA_API hca_status hca_probe_lds_read(int32_t mode, int32_t iters, int32_t grid, uint32_t* sink, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
HCA_API const char* hca_status_string(hca_status status);

/* Library version, e.g. "0.1.0" (static storage). */
HCA_API const char* hca_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HCA_H */
