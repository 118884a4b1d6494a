/*
 * cpdec.h -- context-parallel decode combine on one AMD MI355X (gfx950).
 *
 * The operation is the one described on the page "FlashInfer's
 * Context-Parallel Decode optimisation: Fused A2A + LSE Reduce" (analysis of
 * flashinfer PR #4929):
 *   - section "Introduction": the KV cache of every sequence is split along
 *     the sequence into R shards; decode attention over each shard gives a
 *     partial output o_r and its log-sum-exp lse_r;
 *   - section "Code analysis, 1. Fused kernel": the R partials of each
 *     (sequence, head) are merged with LSE softmax weights, accumulated in
 *     FP32 and converted to FP16/BF16.
 * Here all R shards live in one GPU's memory (one GPU's share of the work
 * after the exchange the page describes); there is no communication.
 *
 * Conventions shared by every entry point
 *   - Plain C ABI.  All tensors are caller-owned device pointers; the library
 *     never allocates, frees or synchronises, and keeps no per-call state.
 *     Its only device state is the static scratch array of
 *     cpdec_cp_decode_noalloc (one per GPU, part of the loaded library).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     CPDEC_OK means the work was enqueued on that stream; device faults
 *     surface at the caller's next synchronisation.
 *   - Every argument check runs before any HIP call; on an error nothing is
 *     enqueued and the outputs are untouched.  The functions never print,
 *     abort or throw.
 *   - Dtypes: CPDEC_F32, CPDEC_F16 (IEEE half), CPDEC_BF16.  Conversions to
 *     F16/BF16 round to nearest even.
 *   - Natural logarithms throughout (lse values are ln of sums of e^score).
 *   - Reentrant and thread-safe; two calls that share a workspace must not
 *     overlap in time on the device (they would race on it).
 */
#ifndef CPDEC_H
#define CPDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPDEC_MAX_SHARDS 64

typedef enum cpdec_status {
  CPDEC_OK = 0,
  CPDEC_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, Hq % Hkv != 0,
                                shard count outside [1, CPDEC_MAX_SHARDS],
                                stride smaller than a row, size overflow    */
  CPDEC_ERR_UNSUPPORTED = 2, /* head_dim or dtype combination not built    */
  CPDEC_ERR_ALIGNMENT = 3,   /* pointer or stride not 16-byte aligned       */
  CPDEC_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned  */
  CPDEC_ERR_HIP = 5          /* the HIP runtime rejected a kernel launch    */
} cpdec_status;

typedef enum cpdec_dtype {
  CPDEC_F32 = 0,
  CPDEC_F16 = 1,
  CPDEC_BF16 = 2
} cpdec_dtype;

/* Shape and layout of one partial-attention call. */
typedef struct cpdec_attn_desc {
  int32_t batch;          /* B  > 0: sequences, one query token each        */
  int32_t num_q_heads;    /* Hq > 0                                          */
  int32_t num_kv_heads;   /* Hkv > 0, Hq % Hkv == 0; query head hq reads kv
                             head hq / (Hq / Hkv)                           */
  int32_t head_dim;       /* D in {64, 128, 256}                             */
  int32_t num_shards;     /* R in [1, CPDEC_MAX_SHARDS]                      */
  int32_t kv_capacity;    /* tokens allocated per (shard, sequence, kv head);
                             every lens entry must be <= kv_capacity.
                             kv_capacity * kv_stride_token * 2 must stay
                             below 2^31 (32-bit offsets within one
                             (shard, sequence, kv head); else UNSUPPORTED)  */
  int64_t kv_stride_batch; /* element strides of each K/V shard tensor;     */
  int64_t kv_stride_head;  /* the D elements of a token are contiguous.     */
  int64_t kv_stride_token; /* [B][Hkv][cap][D] contiguous is
                              (Hkv*cap*D, cap*D, D)                         */
  float sm_scale;         /* softmax scale; 0 selects 1/sqrt(D)             */
  cpdec_dtype qkv_dtype;  /* CPDEC_F16 or CPDEC_BF16 (q, K and V)           */
  cpdec_dtype opart_dtype;/* o_part storage: CPDEC_F32 (recommended), F16,
                             BF16                                           */
  int32_t chunk_tokens;   /* split-KV chunk length in tokens; 0 lets the
                             library pick, otherwise a multiple of 32.  A
                             request is raised to keep at most 256 chunks
                             and lowered to at most 2^18 tokens (each wave
                             accumulates its p.V sums in FP32; longer
                             chunks drift past the output tolerance on
                             inputs where one early token dominates);
                             cpdec_attn_plan reports the length used      */
} cpdec_attn_desc;

/*
 * Bytes of device workspace cpdec_attn_partial needs for `d` (0 when every
 * shard fits one chunk and the launch keeps index order).  Returns 0 for an
 * invalid descriptor as well; such a descriptor is then rejected by
 * cpdec_attn_partial itself.
 *
 * Workspace layout, shared by both attention entry points: the first
 * CPDEC_STEP_COUNTER_BYTES bytes hold arrival counters (cpdec_cp_decode's,
 * and cpdec_attn_partial's when it combines chunks in its launch); they must
 * be zero before the first call on a workspace (cpdec_workspace_clear, once)
 * and every completed call leaves them zero.  Then either the chunk partials
 * (split shards) or the longest-first launch order (32 bytes per (shard,
 * sequence) pair; see cpdec_attn_order), whose contents on entry do not
 * matter.
 */
#define CPDEC_STEP_COUNTER_BYTES 65536
size_t cpdec_attn_workspace_bytes(const cpdec_attn_desc* d);

/*
 * Bytes of device workspace cpdec_cp_decode needs for `d`: the counter region
 * plus the chunk partials, so always at least CPDEC_STEP_COUNTER_BYTES (0 for
 * an invalid descriptor).  A workspace of this size also serves
 * cpdec_attn_partial for the same descriptor.
 */
size_t cpdec_step_workspace_bytes(const cpdec_attn_desc* d);

/*
 * Number of kernel launches cpdec_cp_decode makes for `d`: 1 (the usual case),
 * or 2 to 3 when a limit of the one-launch form is exceeded (see
 * cpdec_cp_decode), one more for the longest-first order pre-pass (see
 * cpdec_attn_order).  Errors: the descriptor checks of cpdec_attn_partial.
 */
cpdec_status cpdec_step_plan(const cpdec_attn_desc* d, int32_t* launches);

/*
 * The launch plan cpdec_attn_partial uses for `d`: the split-KV chunk length
 * in tokens, the number of chunks per (shard, sequence, kv head) and the
 * waves per workgroup.  Any output pointer may be NULL.  Errors: the same
 * descriptor checks as cpdec_attn_partial (INVALID_ARG, UNSUPPORTED,
 * ALIGNMENT); outputs are untouched on error.
 */
cpdec_status cpdec_attn_plan(const cpdec_attn_desc* d, int32_t* chunk_tokens,
                             int32_t* num_chunks, int32_t* waves);

/*
 * Whether calls with `d` launch their work longest first (*longest_first =
 * 1) or in index order (0).  Longest first applies when the library picks the
 * schedule (chunk_tokens == 0), shards are not split, there are at least 2048
 * work units (shards x sequences x kv heads x ceil(G/16)), at most 4096
 * (shard, sequence) pairs and at least 4 GiB of K and V at capacity
 * (shards x sequences x kv heads x kv_capacity x D x 4 bytes; below that the
 * pre-pass, about 10 us, outweighs the gain): a one-workgroup pre-pass kernel
 * sorts the pairs by
 * lens (longest first, ties in index order) into the workspace, and the
 * attention kernel takes its units in that order, so that the short units
 * fill the end of the launch instead of the long ones (ragged batches finish
 * sooner; every output is the same bit for bit either way, since each unit's
 * arithmetic does not depend on when it runs).  The pre-pass is one more
 * launch on the stream.  `longest_first` may be NULL.  Errors: the descriptor
 * checks of cpdec_attn_partial; the output is untouched on error.
 */
cpdec_status cpdec_attn_order(const cpdec_attn_desc* d, int32_t* longest_first);

/*
 * Number of kernel launches cpdec_attn_partial makes for `d` (1 or 2: the
 * order pre-pass, or a chunk-combine launch when the combine does not fit the
 * attention launch).  `launches` may be NULL.  Errors: the descriptor checks
 * of cpdec_attn_partial; the output is untouched on error.
 */
cpdec_status cpdec_attn_launches(const cpdec_attn_desc* d, int32_t* launches);

/*
 * Per-shard decode attention (page section "Introduction").
 *
 * For every shard r, sequence b and query head hq, with L = lens[r*B + b] and
 * g = hq / (Hq/Hkv):
 *     s_t    = sm_scale * <q[b,hq,:], K_r[b,g,t,:]>         for t < L
 *     o_r    = sum_t e^{s_t - m} V_r[b,g,t,:] / sum_t e^{s_t - m},  m = max s
 *     lse_r  = m + ln sum_t e^{s_t - m}
 * and an empty shard (L == 0) gives o_r = 0, lse_r = -inf.  Tokens at
 * positions >= L are never read.
 *
 *   d            host pointer to the descriptor (read during the call)
 *   q            device, [B][Hq][D] contiguous, qkv_dtype, 16-byte aligned
 *   k_shards     host array of R device pointers; shard r's K is
 *                [B][Hkv][kv_capacity][D] under the descriptor's strides
 *   v_shards     same for V (same strides).  Both arrays are read during the
 *                call and not retained.  Every pointer and every stride (in
 *                bytes) must be a multiple of 16.
 *   lens         device, int32 [R][B]; values in [0, kv_capacity].  The
 *                kernels clamp to that range (a negative length counts as
 *                0, one above kv_capacity as kv_capacity), so no value makes
 *                them read outside the shard; they report nothing about it.
 *   o_part       device, [R][B][Hq][D] contiguous, opart_dtype, 16-byte aligned
 *   lse_part     device, float [R][B][Hq]
 *   workspace    device, at least cpdec_attn_workspace_bytes(d) bytes,
 *                256-byte aligned; may be NULL when that size is 0.  Its
 *                counter region (the first CPDEC_STEP_COUNTER_BYTES bytes)
 *                must be zero before the first call on it and is left zero
 *                by every completed call; the rest holds the split-KV chunk
 *                partials or the launch order, and its contents on entry do
 *                not matter (also when one buffer serves descriptors of
 *                different shapes).  Two calls that may run at the same time
 *                need separate workspaces.  When shards are split, the last
 *                chunk workgroup of each (shard, sequence, kv head) combines
 *                that unit's chunks in the attention launch (at most 64
 *                chunks and 1024 such units); beyond that a chunk-combine
 *                launch follows.  The order pre-pass precedes the attention
 *                when the launch is longest first (cpdec_attn_order).
 *                cpdec_attn_launches tells the count.
 *   stream       hipStream_t
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIP (see above).
 */
cpdec_status cpdec_attn_partial(const cpdec_attn_desc* d, const void* q,
                                const void* const* k_shards,
                                const void* const* v_shards,
                                const int32_t* lens, void* o_part,
                                float* lse_part, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * LSE merge of R partials (page section "Code analysis, 1. Fused kernel").
 *
 * For every row n (a (sequence, head) pair):
 *     M      = max_r lse_part[r][n]                (over finite entries)
 *     w_r    = e^{lse_part[r][n] - M}              (shards with -inf skipped:
 *                                                   their o_part rows are
 *                                                   never read)
 *     out[n] = round(sum_r w_r * o_part[r][n][:] / sum_r w_r)
 *     lse_out[n] = M + ln sum_r w_r
 * If every shard of a row is -inf: out[n] = 0 and lse_out[n] = -inf.
 * Weights and the merged lse are formed in FP64, the sum over shards in FP32
 * in shard order, then one rounding to out_dtype.
 *
 *   o_part     device, [R][rows][head_dim] contiguous, in_dtype, 16-byte aligned
 *   lse_part   device, float [R][rows]; entries finite or -inf (NaN and +inf
 *              are outside the contract)
 *   num_shards R in [1, CPDEC_MAX_SHARDS]
 *   rows       >= 0 (0 enqueues nothing); rows * head_dim * sizeof(in) and
 *              num_shards * rows * 4 must stay below 2^31 (32-bit offsets
 *              within one shard; else UNSUPPORTED)
 *   head_dim   in {64, 128, 256, 512}
 *   in_dtype   CPDEC_F32, CPDEC_F16 or CPDEC_BF16
 *   out_dtype  CPDEC_F32, CPDEC_F16 or CPDEC_BF16
 *   out        device, [rows][head_dim], out_dtype, 16-byte aligned
 *   lse_out    device, float [rows], or NULL to skip writing it
 *   stream     hipStream_t
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, HIP.
 */
cpdec_status cpdec_lse_merge(const void* o_part, const float* lse_part,
                             int32_t num_shards, int64_t rows, int32_t head_dim,
                             cpdec_dtype in_dtype, cpdec_dtype out_dtype,
                             void* out, float* lse_out, void* stream);

/*
 * The whole step: cpdec_attn_partial's partials (o_part/lse_part, same
 * values to FP32 rounding) and their LSE merge into out/lse_out with the merge
 * formula of cpdec_lse_merge (page sections "Introduction" and "Code
 * analysis, 1. Fused kernel"), normally in ONE kernel launch: every
 * workgroup hands its partial over through device-scope stores and an
 * arrival counter per (sequence, kv head); the last workgroup of each such
 * group combines its shards' chunks, writes o_part/lse_part and merges the
 * shards.  The result does not depend on which workgroup arrives last.
 * The one-launch form needs a group that one workgroup can merge with one
 * round of loads: groups (sequences x kv heads x ceil(G/16)) <= 1024, o_part
 * below 2 GiB, and either unsplit shards (at most 8 shards, min(G,16) x D/4
 * <= the workgroup's threads, at most 1024 workgroups) or split shards (at
 * most 16 chunks, shards x min(G,16) x D/4 <= the workgroup's threads).
 * Split groups beyond that still take one launch in two levels -- the last
 * chunk workgroup of each (shard, sequence, kv head) combines its chunks,
 * the last of the group's shards merges them -- when min(G,16) x D/4 <= the
 * workgroup's threads, at most 64 chunks and units + groups <= 1024.
 * Otherwise the step runs as separate launches: the attention, then -- when a
 * query head's shards x chunks (chunks rounded up to a power of two) are at
 * most 64 -- one kernel that combines the chunks and merges the shards per
 * (sequence, query head), else a chunk-combine and a merge launch; the order
 * pre-pass of cpdec_attn_order goes in front when it applies (cpdec_step_plan
 * tells how many launches).
 * `out` agrees with cpdec_lse_merge of the same partials to rounding.
 *
 *   d, q, k_shards, v_shards, lens, o_part, lse_part, stream
 *              as for cpdec_attn_partial
 *   out        device, [B][Hq][D] in qkv_dtype, 16-byte aligned
 *   lse_out    device, float [B][Hq], or NULL to skip writing it
 *   workspace  device, at least cpdec_step_workspace_bytes(d) bytes, 256-byte
 *              aligned.  Its first CPDEC_STEP_COUNTER_BYTES bytes must be zero
 *              before the first call on it (cpdec_workspace_clear does that
 *              once, after allocation); every call that completes leaves them
 *              zero again, whatever the shape.  The rest is scratch.  Two calls
 *              that may run at the same time need separate workspaces.
 * Errors: as cpdec_attn_partial; INVALID_ARG for a NULL out; ALIGNMENT for a
 * misaligned out or lse_out; WORKSPACE for a missing or short workspace;
 * UNSUPPORTED when the step needs separate launches and B x Hq x D x
 * (o_part element bytes) or R x B x Hq x 4 reaches 2 GiB (the merge kernel's
 * 32-bit offsets, as for cpdec_lse_merge).
 */
cpdec_status cpdec_cp_decode(const cpdec_attn_desc* d, const void* q,
                             const void* const* k_shards,
                             const void* const* v_shards, const int32_t* lens,
                             void* o_part, float* lse_part, void* out,
                             float* lse_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * cpdec_cp_decode for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc: the same step, kernels and results (bit for bit), but its
 * scratch (arrival counters, chunk partials, launch order) lives in a
 * static device array of CPDEC_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held until the process ends.  The caller passes inputs and
 * outputs only; nothing is allocated or freed, by the library or for it.
 *
 * The first call on a device looks up that GPU's array (the device `stream`
 * belongs to; the current device for the null stream) and clears its counter
 * region with a kernel on `stream`;
 * every completed call leaves the counters zero again, and the rest of the
 * array is overwritten before it is read.  Every call on one GPU shares the
 * array: two calls that may overlap in time on the same GPU (other streams,
 * other threads) race on it and must be serialised by the caller, e.g. by
 * issuing them on one stream.
 *
 *   d, q, k_shards, v_shards, lens, o_part, lse_part, out, lse_out, stream
 *              as for cpdec_cp_decode
 * Errors: as cpdec_cp_decode (checked before any HIP call); WORKSPACE when
 * the step needs more scratch than CPDEC_NOALLOC_SCRATCH_BYTES
 * (cpdec_step_workspace_bytes(d) tells how much it needs); HIP when the
 * array cannot be reached on the current device.
 */
#define CPDEC_NOALLOC_SCRATCH_BYTES (16u << 20)
cpdec_status cpdec_cp_decode_noalloc(const cpdec_attn_desc* d, const void* q,
                                     const void* const* k_shards,
                                     const void* const* v_shards, const int32_t* lens,
                                     void* o_part, float* lse_part, void* out,
                                     float* lse_out, void* stream);

/*
 * Zero-fill `bytes` bytes of a buffer on `stream` with a kernel (no
 * hipMemset, so it is safe to record in a HIP graph).  A new workspace needs
 * it once, for its counter region (the first CPDEC_STEP_COUNTER_BYTES bytes),
 * before its first use by either attention entry point.  `workspace` must be
 * 256-byte aligned.  Errors: INVALID_ARG, ALIGNMENT, HIP.
 */
cpdec_status cpdec_workspace_clear(void* workspace, size_t bytes, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* cpdec_status_string(cpdec_status s);

/* Library version string, e.g. "cpdec 0.1.0 gfx950". */
const char* cpdec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPDEC_H */
