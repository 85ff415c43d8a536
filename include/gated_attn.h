/*
 * gated_attn.h -- C ABI of the MI355X (gfx950) gated grouped-query attention
 * library (libgated_attn.so).
 *
 * The operation (cuDNN FE-OSS "Gated Attention Block (SM107)", Overview,
 * stages (4) and (5); FreeToken PR #781, Summary, for the bf16 rounding chain):
 *
 *     O   = softmax(q K^T * scale) V          fp32 accumulation on the GPU
 *     out = bf16( bf16(O) * bf16(sigmoid(gate)) )   each rounding to nearest even
 *
 * with grouped-query attention: query head h reads kv head h / (H_q / H_kv).
 * A padded slot (sequence length <= 0) produces out = +0 (ROCm/ATOM PR #838,
 * "PAD_SLOT_ID (-1) handling"; cuDNN page, fuse_gate "dead-row select").
 *
 * Conventions shared by every entry point (cuDNN page, Forward: one caller-owned
 * workspace, nothing allocated, nothing read back to the host, every stage on
 * the one stream given; Requirements: unsupported cases are declined with a
 * typed error rather than served slowly):
 *   - bf16 tensors are passed as pointers to their 16-bit patterns (uint16_t).
 *   - Every pointer is a device pointer owned by the caller.  The library never
 *     allocates, frees, synchronises or copies device memory to the host, so a
 *     call can be captured into a HIP graph.  Inputs are never written.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL means the null
 *     stream).  A call returns once the work is enqueued, not when it is done.
 *   - Every argument the host can see is checked before anything is launched;
 *     on any status other than GA_OK nothing has been enqueued and no memory
 *     has been touched.  Values that live only in device memory (sequence
 *     lengths, page ids) are preconditions and are not checked.
 *   - All tensors are dense, contiguous, row-major, and 16-byte aligned
 *     (block_table / seq_lens: 4-byte aligned).
 */
#ifndef GATED_ATTN_H
#define GATED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ga_status {
    GA_OK = 0,
    GA_ERR_INVALID_ARGUMENT = 1,    /* null/misaligned pointer, bad size or scale */
    GA_ERR_UNSUPPORTED = 2,         /* valid but not served: device, head dim, group size */
    GA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < gated_attn_decode_workspace_size() */
    GA_ERR_HIP = 4                  /* the HIP runtime reported an error; see gated_attn_last_hip_error() */
} ga_status;

/* GQA groups (both entry points).  Query head h attends with kv head
 * h / G, G = H_q / H_kv (contiguous groups: cuDNN "Gated Attention Block",
 * Overview, stage (4), GQA H_q / H_kv).  Served: G = 1..16 -- among them the
 * h_q = 32, h_kv = 2 geometry of that page's Performance section and the
 * non-power-of-two groups the FreeToken PR #781 tests (Correctness and actual
 * execution).  Decode serves a whole group in one workgroup; prefill runs
 * G = 9..16 as two workgroups per kv head (ceil(G/2) and floor(G/2) heads),
 * each streaming that head's K/V.  G > 16: GA_ERR_UNSUPPORTED; H_q not a
 * multiple of H_kv: GA_ERR_INVALID_ARGUMENT. */

/* Shape of a paged decode call. */
typedef struct ga_decode_dims {
    int32_t batch;             /* B >= 0 sequences, one query token each */
    int32_t num_q_heads;       /* H_q */
    int32_t num_kv_heads;      /* H_kv, dividing H_q; see GQA groups below */
    int32_t head_dim;          /* D; must be 256 */
    int32_t page_size;         /* tokens per page: 16, or 1 (every table entry is a token slot) */
    int32_t max_pages_per_seq; /* W: columns of block_table (the allocated capacity) */
    int64_t num_pages;         /* P: pages in each of k_pool / v_pool */
} ga_decode_dims;

/* How a decode call splits each sequence.  The grid, NS and the workspace are
 * chosen from the dims alone, i.e. from the allocated capacity W * page_size
 * and not from the current lengths, so one captured graph serves every length
 * up to the capacity (FreeToken PR #781, Automatic dispatch, ties its
 * dispatch to the allocated capacity).  On the device, each sequence's visible
 * keys (from the window start, rounded down to a page, to its length) are cut
 * into NS equal page-aligned parts of at least 64 tokens, so a sequence far
 * shorter than the capacity still spreads over its NS blocks.  When the grid
 * holds more blocks than one round (B * H_kv * NS above 256), a sequence cut in
 * two gives its first part about 11/16 of the keys (at most T). */
typedef struct ga_decode_plan {
    int32_t tokens_per_split;  /* T: the most tokens one (sequence, kv head, split) block covers */
    int32_t num_splits;        /* NS = ceil(W * page_size / T) blocks per (sequence, kv head) */
    size_t workspace_bytes;    /* fp32 partials: B * H_q * num_splits * (D + 2) * 4, rounded up */
} ga_decode_plan;

/* Fill *plan for dims.  GA_ERR_INVALID_ARGUMENT / GA_ERR_UNSUPPORTED as
 * gated_attn_decode would return for these dims (GA_ERR_UNSUPPORTED also when
 * a grid would exceed one launch: more than 2^22 stage-1 workgroups, i.e.
 * B * H_kv * num_splits > 2^22, or B * H_q > 2^25; nothing else bounds B). */
ga_status gated_attn_decode_plan(const ga_decode_dims *dims, ga_decode_plan *plan);

/* Bytes of device workspace gated_attn_decode needs for dims (0 if dims are
 * invalid or batch == 0). */
size_t gated_attn_decode_workspace_size(const ga_decode_dims *dims);

/*
 * Gated GQA decode over a paged bf16 KV pool: split-KV partial attention
 * (FreeToken PR #781, Summary: stage1, then a stage2 fp32 reduction) followed,
 * in the same second kernel, by the bf16 rounding of O, the bf16 sigmoid of the
 * gate and the rounded product -- two kernel launches per call, none of them
 * for the gate.  At page size 1 the first launch addresses token rows by
 * 32-bit offsets from the pool's start, or by 64-bit addresses when the pool's
 * rows span more than 4 GiB (chosen from num_pages alone; the results are
 * identical either way).
 *
 *   q, gate     [B][H_q][D]                       bf16, read
 *   k_pool,
 *   v_pool      [num_pages][page_size][H_kv][D]   bf16, read
 *   block_table [B][max_pages_per_seq]            int32 page ids, read; any
 *               entry of row b may be read (they are loaded before the length
 *               is known), but the values at or past ceil(seq_lens[b] /
 *               page_size) are ignored: they may hold anything (e.g. -1)
 *   seq_lens    [B]                               int32 KV lengths, read;
 *               <= 0 marks a padded slot (its output row is +0)
 *   scale       softmax scale (finite, > 0), e.g. 1/sqrt(D)
 *   out         [B][H_q][D]                       bf16, written
 *   workspace   >= gated_attn_decode_workspace_size(dims) bytes, 16-byte
 *               aligned, contents need not be initialised; overwritten
 *
 * Preconditions in device memory (not checked): 0 <= seq_lens[b] <=
 * max_pages_per_seq * page_size, and every block_table entry that is read is
 * in [0, num_pages).  A violation gives an unspecified output row, never an
 * access outside the buffers: the kernels clamp lengths to the capacity and
 * page ids into [0, num_pages).  Concurrent calls must not share a workspace.
 */
ga_status gated_attn_decode(const uint16_t *q, const uint16_t *gate, const uint16_t *k_pool,
                            const uint16_t *v_pool, const int32_t *block_table,
                            const int32_t *seq_lens, float scale, uint16_t *out, void *stream,
                            const ga_decode_dims *dims, void *workspace, size_t workspace_bytes);

/* Bytes of device memory gated_attn_decode_noalloc keeps per GPU for the
 * split partials (16 MiB). */
#define GA_DECODE_SCRATCH_BYTES (16u << 20)

/*
 * gated_attn_decode for callers that cannot allocate device memory or pass a
 * workspace -- code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same operation, kernels, arguments (minus the
 * workspace) and errors as gated_attn_decode; the split partials go to a
 * device array of GA_DECODE_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends.  Nothing is allocated or freed by the
 * call; its first call on a device looks up that device's array (call it
 * once outside graph capture first).
 *   GA_ERR_WORKSPACE_TOO_SMALL when gated_attn_decode_workspace_size(dims) >
 *   GA_DECODE_SCRATCH_BYTES (e.g. B = 224 at a 6,144-token capacity needs
 *   7.4 MB and fits; B * H_q * num_splits past about 16,000 rows does not).
 * Every call on one GPU shares that GPU's array and leaves its partials
 * there; nothing in it needs to start at zero (stage 1 writes every partial
 * stage 2 reads in the same call).  Calls that overlap on one GPU -- on
 * streams not ordered with each other -- race on the array and must not be
 * issued.
 */
ga_status gated_attn_decode_noalloc(const uint16_t *q, const uint16_t *gate,
                                    const uint16_t *k_pool, const uint16_t *v_pool,
                                    const int32_t *block_table, const int32_t *seq_lens,
                                    float scale, uint16_t *out, void *stream,
                                    const ga_decode_dims *dims);

/* Measurement hook for benchmarks: reads `bytes` of device memory at `src`
 * once, with the non-temporal 16-byte loads the decode's K/V stream uses, in
 * one kernel launch on `stream`, so a caller can time the device's streaming-
 * read rate beside the decode's KV bandwidth.  Not part of the attention path.
 *   src    device buffer, 16-byte aligned, read
 *   bytes  a multiple of 16 (0: nothing is launched)
 *   sink   device uint32[1], 4-byte aligned; written only if the XOR of all
 *          words read equals 0x9e3779b9 (it keeps the loads from being removed)
 * GA_ERR_INVALID_ARGUMENT for a NULL or misaligned pointer or a size not a
 * multiple of 16; GA_ERR_UNSUPPORTED off gfx950; GA_ERR_HIP on a launch error. */
ga_status gated_attn_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Shape of a dense prefill call: S_q = S_kv = seq_len. */
typedef struct ga_prefill_dims {
    int32_t batch;        /* B >= 0 */
    int32_t seq_len;      /* S >= 0 */
    int32_t num_q_heads;  /* H_q */
    int32_t num_kv_heads; /* H_kv, dividing H_q; see GQA groups below */
    int32_t head_dim;     /* D; must be 256 */
} ga_prefill_dims;

/*
 * Gated dense prefill attention with bf16 matrix-core (MFMA) products and the
 * same gate epilogue (cuDNN page, Forward: fuse_gate folds stage (5) into the
 * SDPA epilogue), one kernel launch per call.
 *
 *   q, gate, out  [B][S][H_q][D]   bf16 (q, gate read; out written)
 *   k, v          [B][S][H_kv][D]  bf16, read
 *   causal        non-zero: query i sees keys j <= i; zero: every key
 *
 * All buffers 16-byte aligned and device-resident, owned by the caller; out
 * is written in full.  GA_ERR_INVALID_ARGUMENT for a NULL or misaligned
 * pointer, negative sizes or a scale that is not finite and positive;
 * GA_ERR_UNSUPPORTED for D != 256, groups above 16, a device other than
 * gfx950, one sequence's K (or V) rows spanning more than 2^31 - 1 bytes
 * (S * H_kv * D * 2), or more than 2^22 workgroups (B * H_kv * parts *
 * ceil(S / 16), parts = 2 for groups above 8, else 1).  B = 0 or S = 0 does
 * nothing and returns GA_OK.
 */
ga_status gated_attn_prefill(const uint16_t *q, const uint16_t *gate, const uint16_t *k,
                             const uint16_t *v, float scale, int causal, uint16_t *out,
                             void *stream, const ga_prefill_dims *dims);

/*
 * Attention-spec options of the _ex entry points.  The pages name these
 * options without defining them: the FreeToken PR #781 keeps windows and sinks
 * off its fused path (Automatic dispatch) and tests them (Correctness and
 * actual execution); the cuDNN "Gated Attention Block" page's Forward offers
 * return_lse (softmax statistics [B, H_q, S] fp32) and seq_lens_present
 * (per-batch KV lengths).  This library reads them as follows, per query row:
 *   visible keys  decode: j < L; prefill row i: j < kv_lens[b], j <= i if
 *                 causal; and with window w > 0 only the w most recent of
 *                 them (decode: j >= L - w; prefill: j > i - w)
 *   Z             sum over visible j of exp(s_j), plus exp(sinks[h]) if sinks
 *   O             sum over visible j of exp(s_j) V_j / Z   (s_j = scale q.k_j)
 *   lse           ln Z, natural log; -inf when Z = 0
 *   A row with no visible key is dead and gets out = +0 (its lse is the sink
 *   logit, or -inf).  A zeroed struct (or NULL) is plain attention.
 * All pointers are device pointers, 4-byte aligned, owned by the caller.
 */
typedef struct ga_attn_options {
    const float *sinks;     /* [H_q] fp32 sink logits (natural-log units, not scaled), or NULL */
    float *lse;             /* written: decode [B][H_q], prefill [B][S][H_q] fp32; or NULL */
    const int32_t *kv_lens; /* prefill only, [B] int32 key lengths (clamped to [0, S]);
                               NULL = S for every sequence; must be NULL for decode */
    int32_t window;         /* > 0: sliding window of that many keys; <= 0: none */
    int32_t flags;          /* reserved; must be 0 */
} ga_attn_options;

/* gated_attn_decode with options appended (the cuDNN page's Forward appends
 * new arguments at the end).  opts == NULL is gated_attn_decode.  Extra
 * errors: GA_ERR_INVALID_ARGUMENT for flags != 0, a misaligned pointer, or
 * kv_lens set.  The workspace size does not depend on the options. */
ga_status gated_attn_decode_ex(const uint16_t *q, const uint16_t *gate, const uint16_t *k_pool,
                               const uint16_t *v_pool, const int32_t *block_table,
                               const int32_t *seq_lens, float scale, uint16_t *out, void *stream,
                               const ga_decode_dims *dims, void *workspace,
                               size_t workspace_bytes, const ga_attn_options *opts);

/*
 * Gated GQA decode over FP8 K / V pools: each element is an OCP float8 e4m3
 * code (1 sign, 4 exponent bits biased by 7, 3 fraction bits, no infinities)
 * and K = k_descale * value(code), V = v_descale * value(code) with one factor
 * per tensor (the cuDNN "Gated Attention Block" page's FP8 pipeline takes
 * static per-tensor scales, Forward: Quantization specs).  Everything else --
 * layouts ([num_pages][page_size][H_kv][D], one byte per element; page size
 * 16, or 1 with block-table entries as token slots), q, gate,
 * out, dims, plan, workspace, options, errors -- is as gated_attn_decode_ex.
 * The factors must be finite and > 0 (else GA_ERR_INVALID_ARGUMENT).  The K
 * factor is folded into the score scale and the V factor into O before its
 * bf16 rounding; the codes themselves are decoded exactly.
 */
ga_status gated_attn_decode_fp8kv(const uint16_t *q, const uint16_t *gate, const uint8_t *k_pool,
                                  const uint8_t *v_pool, const int32_t *block_table,
                                  const int32_t *seq_lens, float scale, float k_descale,
                                  float v_descale, uint16_t *out, void *stream,
                                  const ga_decode_dims *dims, void *workspace,
                                  size_t workspace_bytes, const ga_attn_options *opts);

/*
 * Gated GQA decode with CSR token indexing at page size 1, the serving layout
 * of the FreeToken PR #781 (Automatic dispatch: a CSR index of allocated
 * capacity; the server runs with page size 1): sequence b's tokens are
 * kv_indices[kv_indptr[b]] .. kv_indices[kv_indptr[b + 1] - 1], each a row of
 * the pools k_pool / v_pool [num_pages][1][H_kv][D] (num_pages = pool rows).
 * Its length is kv_indptr[b + 1] - kv_indptr[b] (no seq_lens).
 *   kv_indptr      [B + 1] int32, device, non-decreasing
 *   kv_indices     [index_capacity] int32, device
 *   dims           page_size must be 1; max_pages_per_seq is the per-sequence
 *                  capacity in tokens, which alone fixes the plan and workspace
 * Everything else as gated_attn_decode_ex.  Row pointers outside
 * [0, index_capacity], lengths past the capacity and slots outside the pools
 * are clamped (an unspecified row, never an access outside the buffers).
 * GA_ERR_INVALID_ARGUMENT for null or misaligned index arrays or a negative
 * capacity; GA_ERR_UNSUPPORTED for page_size != 1.
 */
ga_status gated_attn_decode_csr(const uint16_t *q, const uint16_t *gate, const uint16_t *k_pool,
                                const uint16_t *v_pool, const int32_t *kv_indptr,
                                const int32_t *kv_indices, int64_t index_capacity, float scale,
                                uint16_t *out, void *stream, const ga_decode_dims *dims,
                                void *workspace, size_t workspace_bytes,
                                const ga_attn_options *opts);

/*
 * gated_attn_decode_csr over e4m3 pools: the CSR token indexing of
 * gated_attn_decode_csr with the e4m3 codes and per-tensor factors of
 * gated_attn_decode_fp8kv (k_pool / v_pool [num_pages][1][H_kv][D], one byte
 * per element).  Arguments, ownership and errors as those two entry points.
 */
ga_status gated_attn_decode_fp8kv_csr(const uint16_t *q, const uint16_t *gate,
                                      const uint8_t *k_pool, const uint8_t *v_pool,
                                      const int32_t *kv_indptr, const int32_t *kv_indices,
                                      int64_t index_capacity, float scale, float k_descale,
                                      float v_descale, uint16_t *out, void *stream,
                                      const ga_decode_dims *dims, void *workspace,
                                      size_t workspace_bytes, const ga_attn_options *opts);

/* gated_attn_prefill with options appended.  opts == NULL is
 * gated_attn_prefill.  GA_ERR_INVALID_ARGUMENT for flags != 0 or a misaligned
 * pointer.  Key lengths mask keys only: a row past its sequence's length
 * still attends to the sequence's keys (causal rows see all of them). */
ga_status gated_attn_prefill_ex(const uint16_t *q, const uint16_t *gate, const uint16_t *k,
                                const uint16_t *v, float scale, int causal, uint16_t *out,
                                void *stream, const ga_prefill_dims *dims,
                                const ga_attn_options *opts);

/* Shape of a QK-norm / RoPE call over T tokens. */
typedef struct ga_qk_norm_rope_dims {
    int64_t num_tokens;    /* T >= 0 */
    int32_t num_q_heads;   /* H_q */
    int32_t num_kv_heads;  /* H_kv */
    int32_t head_dim;      /* D; must be 256 */
    int32_t rope_dim;      /* R: rotated leading dims of every head, 0..D, a multiple of 8 */
    int32_t page_size;     /* pool page size (must be 16) when slot_mapping is given */
    int32_t reserved;      /* ignored */
    int64_t num_pages;     /* pages of k_out / v_out when slot_mapping is given */
} ga_qk_norm_rope_dims;

/*
 * The step before attention (cuDNN "Gated Attention Block" page, Overview
 * stages (2)+(3), one kernel for Q and K; Weights and tables: cos / sin
 * rotary tables in the activation dtype, rotate-half on the first rope_dim
 * dims of every head, norm weights [D]): for every head row x of q and k,
 *   y = x / sqrt(mean(x^2) + eps) * w       (w_q_norm / w_k_norm; both NULL: y = x)
 *   z_i = y_i cos[t][i] - y_{i+R/2} sin[t][i],  z_{i+R/2} = y_{i+R/2} cos[t][i+R/2]
 *         + y_i sin[t][i+R/2]  for i < R/2;  z_d = y_d for d >= R
 * computed in fp32 and rounded once to bf16 (the page's fused form normalises
 * and rotates on fp32 values and writes once).  MRoPE and any other position
 * scheme is expressed through the per-token tables.
 *   q, q_out   [T][H_q][D] bf16      k, v  [T][H_kv][D] bf16     cos, sin [T][R] bf16
 * With slot_mapping ([T] int64, device): token t's K (normed and rotated) and
 * V go to slot s = slot_mapping[t] of the pools k_out / v_out
 * ([num_pages][16][H_kv][D]; slot s is page s / 16, row s % 16); s < 0 or
 * s >= num_pages * 16 writes nothing.  Without it: k_out is dense [T][H_kv][D]
 * and v_out is a dense copy of v, or NULL (not written).
 * Errors: GA_ERR_INVALID_ARGUMENT for null or misaligned pointers (16 bytes;
 * slot_mapping 8),
 * one norm weight without the other, eps < 0 or not finite, odd R, missing
 * tables with R > 0; GA_ERR_UNSUPPORTED for D != 256, R not a multiple of 8,
 * page size != 16, T * (H_q + H_kv) > 2^30, or a non-gfx950 device.  One
 * kernel launch on `stream`; nothing allocated.  Inputs are not written
 * (q_out may not alias q, nor the pools k / v).
 */
ga_status gated_attn_qk_norm_rope(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  const uint16_t *w_q_norm, const uint16_t *w_k_norm, float eps,
                                  const uint16_t *cos, const uint16_t *sin,
                                  const int64_t *slot_mapping, uint16_t *q_out, uint16_t *k_out,
                                  uint16_t *v_out, void *stream, const ga_qk_norm_rope_dims *dims);

/* Static, human-readable name of a status. */
const char *gated_attn_status_string(ga_status status);

/* The hipError_t value behind the calling thread's most recent GA_ERR_HIP
 * (0 if none). */
int gated_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GATED_ATTN_H */
