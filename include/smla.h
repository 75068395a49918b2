/*
 * smla.h -- sparse MLA decode and the split-KV LSE merge on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named as device memory must be a device pointer that the
 * caller allocated and owns; the library never allocates, frees or synchronizes.  Calls are
 * asynchronous and ordered on the given HIP stream (0 = the null stream).  Arguments are
 * checked on the host before anything is launched; on an error nothing is written.
 *
 * Method (cited by page title and section; the pages are API documentation pages of vLLM):
 *   sparse_mla_cute page, "What this module computes": each query token t and head h attends
 *     over its own set of FP8 (E4M3) KV rows, the active columns c of the token
 *     (c < lens[t] and indices[t, c] >= 0):
 *       s_c = bmm1 * q[t,h] . kv[c];  out[t,h] = bmm2 * sum_c e^{s_c-m} v_c / (sum_c e^{s_c-m}
 *       + e^{sink_h - m}), m the maximum of the scores and the sink, V the first 512 bytes of
 *       the same row; columns below split_col index pool A, the others pool B; a token with no
 *       active column gets zeros.
 *   attn_sparse page (Kimi K3.1 SparseDcpDecode), module docstring: 576-byte rows (512 latent
 *     + 64 rope bytes) of a per-tensor-scaled FP8 cache; softmax in base 2 with P quantized to
 *     E4M3 at 448 of the running row maximum (RN, satfinite), FP32 sums of the unquantized P,
 *     FP32 accumulation, one BF16 rounding of the output; rows of count 0 give zeros and
 *     LSE -inf; the split partials are merged in FP32 (merge method: weights exp2(max_c - max),
 *     BF16(sum * k_scale / total), LSE = max + log2(total / 448), natural log in the
 *     non-push output).
 *   dcp page, DcpValue.merge: LSE-weighted merge of D split partials in FP32, weights
 *     exp2(lse - top) / sum, empty sources weighted 0, one BF16 rounding.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
typedef int32_t smla_status;
#define SMLA_OK 0
#define SMLA_EINVAL 1        /* a null pointer, bad size, misalignment or bad flag */
#define SMLA_EUNSUPPORTED 2  /* a shape this build has no kernel for (see each entry point) */
#define SMLA_EWORKSPACE 3    /* the workspace is missing or smaller than required */
#define SMLA_EHIP 4          /* a HIP runtime error (device query or kernel launch) */
#define SMLA_ESCRATCH 5      /* sparse_mla_decode_noalloc: the problem's workspace would exceed
                                SMLA_NOALLOC_SCRATCH_BYTES */

/* Flags. */
#define SMLA_LSE_LOG2 0x1u   /* LSE outputs in base 2 (default: natural log) */
#define SMLA_P_ONE_TERM 0x2u /* sparse_mla_decode: P as one E4M3 term (the attn_sparse page's
                                recipe, anchored as described under sparse_mla_decode).
                                Default: two E4M3 terms, P = hi + lo/16 with hi = E4M3(P) and
                                lo = E4M3(16 (P - hi)), which keeps the E4M3 quantization but
                                reaches FP32-level accuracy (relative output error ~1e-3
                                instead of ~2e-2). */
#define SMLA_P_CHUNK_LOCAL 0x4u /* sparse_mla_decode: the chunk-local recipe of the
                                sparse_mla_cute page ("How."): each 128-column window of a
                                token's columns, [128 k, 128 k + 128) of its clamped count, is
                                one key range with its own softmax, P = E4M3(256 x 2^(s2 - m_k))
                                at the window's own maximum m_k (one E4M3 term; no running
                                maximum), FP32 sums of the unquantized P; the windows then merge
                                as split partials with weights 2^(m_k - M), the sink weighted
                                256 x 2^(sink2 - M), LSE2 = M - 8 + log2 L.  The plan must
                                have tiles = 2 and splits = ceil(W / 128) (smla_decode_plan
                                gives such a plan when passed this flag), else
                                SMLA_EUNSUPPORTED.  SMLA_P_ONE_TERM is implied. */

/* The launch decomposition of one sparse_mla_decode call.  A workgroup takes one token, a
 * group of `tiles` 32-head tiles (heads padded up to a multiple of 32) and one of `splits`
 * contiguous ranges of the token's clamped count (range s = [min(n, s*per), +min(n - first,
 * per)), per = ceil(n / splits), as the attn_sparse page's key split); the ranges run in chunks
 * of `chunk` columns and, when splits > 1, their partials (FP32 accumulators with the range's
 * running maximum m and sum l) are merged in FP32, in range order, with weights 2^(m_s - M)
 * (the attn_sparse page's module docstring, "Precision", and its merge method). */
typedef struct smla_plan {
    int32_t splits; /* 1 .. 64 */
    int32_t tiles;  /* 32-head tiles per workgroup: 1 (32 heads, rows loaded into registers) or
                       2 (64 heads, rows gathered straight into LDS; the last group is padded
                       when ceil(H / 32) is odd; ranges of at most 2048 columns,
                       ceil(W / splits) <= 2048, else SMLA_EUNSUPPORTED) */
    int32_t chunk;  /* columns per gathered chunk (64 in this build; output only) */
    int32_t merge;  /* how the split partials are merged (ignored when splits == 1):
                       SMLA_MERGE_LAST: the last range of a (token, head group) to finish merges
                       every column; any grid size.
                       SMLA_MERGE_SPREAD: range s merges the output columns of 32-column tiles
                       [16 s / splits, 16 (s + 1) / splits) of every head (512 / splits columns
                       when splits divides 16), so the merge's reads are spread over all the
                       ranges' workgroups.  The ranges of a (token, head group) wait for each other
                       (a bounded wait, as under sparse_mla_decode), so every workgroup must be
                       resident at once: tiles must be 2 (the 64-head kernel; the 32-head
                       kernel has no spread merge), splits 2 to 16 and the grid, tokens x
                       head groups x splits, at most the device's compute-unit count (one
                       workgroup fits per compute unit), else SMLA_EUNSUPPORTED.  Kernels that
                       run concurrently on other streams may delay some of the workgroups until
                       they finish; a kernel that itself waits on this call's results while
                       holding compute units could make the wait give up. */
    int32_t heads;  /* real heads per workgroup: 0 for 32 x tiles; with tiles = 2 also 16 or 32
                       (the 64-head kernel still runs its two 32-head tiles, the heads past
                       that count as padding that is neither exchanged nor written, so that a
                       small batch spreads over more workgroups with shorter chunk chains and
                       smaller split exchanges); head groups per token = ceil(H / heads). */
} smla_plan;

#define SMLA_MERGE_LAST 0
#define SMLA_MERGE_SPREAD 1

/* The plan sparse_mla_decode uses for these sizes when it is given none: the cheapest, by a
 * predicted time, of every plan the kernels take for them -- the 64-head kernel with 64, 32 or
 * 16 real heads per workgroup over one key range, two ranges under SMLA_MERGE_LAST, or 2 to 16
 * ranges under SMLA_MERGE_SPREAD (grid within the compute units, queried once per
 * device), and the 32-head kernel over 1, 2, 4 or 8 ranges under SMLA_MERGE_LAST.  The
 * prediction is a linear model of the call's time in its workgroup rounds, chunks per range,
 * compute-unit occupancy, heads per workgroup and split-exchange bytes, with coefficients
 * measured on MI355X; ties keep the wider head groups.  Returns SMLA_EINVAL for bad sizes,
 * SMLA_EHIP if the device cannot be queried. */
smla_status smla_decode_plan(int32_t T, int32_t H, int32_t W, int32_t row_bytes, uint32_t flags,
                             smla_plan *plan);

/* Workspace bytes sparse_mla_decode needs under `plan` (0 when plan->splits == 1).  The caller
 * sizes and allocates it once, before any graph capture, and reuses it across calls that are
 * stream ordered (the dcp page, stock_decode: a split-KV workspace sized before capture, shared
 * by stream-ordered calls, no per-call allocation).  Layout:
 *   bytes [0, 4)    status word, int32: the number of (token, head group) split merges that gave
 *                   up waiting for the other key ranges' partials since the workspace was last
 *                   zero-filled (0 in normal operation; see sparse_mla_decode);
 *   bytes [16, ..)  arrival counters, two int32 per token and head group, then padding to a
 *                   multiple of 256 bytes;
 *   then            FP32 partials [T, groups, splits, 32 tiles, 512] (each range's accumulators
 *                   at 448 of its running maximum, not normalized, in the kernel's register
 *                   order) and FP32 (m, l) pairs [T, groups, splits, 32 tiles, 2] (running
 *                   maximum in base 2, sum of the unquantized P), groups = ceil(H / w) with
 *                   w = heads, or 32 x tiles when heads is 0 (slots of 32 x tiles heads; only
 *                   the group's real heads are written and read).
 * Returns 0 for a bad plan. */
size_t smla_decode_workspace_size(const smla_plan *plan, int32_t T, int32_t H);

/*
 * sparse_mla_decode -- sparse MLA decode of T tokens (formula above).
 *
 *   q            device, E4M3 bytes; head h of token t at q + t*q_stride_t + h*q_stride_h,
 *                qk_dim bytes.  16-byte aligned; both strides multiples of 16.
 *   kv_a, rows_a device, pool A: rows_a rows of row_bytes bytes, 16-byte aligned.
 *   kv_b, rows_b device, pool B (may be NULL: then every column uses pool A and split_col is
 *                ignored).  Columns c >= split_col use pool B.
 *   row_bytes    576 (E4M3: 512 latent + 64 rope) or 512 (E4M3 latent): V is bytes
 *                [0, 512) of a row.  Or 656: an fp8_ds_mla row (the dsa_indexer page's 656-byte
 *                MLA cache entry of [kv_c_normed | k_pe], viewed as FP8, FP32 and BF16), read as
 *                the E4M3 latent at bytes [0, 512), one FP32 scale per 128 latent elements at
 *                [512, 528) and the 64-element BF16 rope at [528, 656): K = [latent x scale |
 *                rope], V = latent x scale.  656-byte rows need qk_dim = 576 (q's 64 rope bytes
 *                E4M3 as before) and tiles = 2 (else SMLA_EINVAL / SMLA_EUNSUPPORTED); their
 *                P.V product runs in BF16 (V x scale rounded to BF16, P's E4M3 terms exact).
 *   qk_dim       576 or 512, <= row_bytes: the elements of q and of each row in the score.
 *   indices      device int32 [T, W] row-major: storage rows, negative = unused column.
 *                Every active entry must be < the row count of its pool (precondition, not
 *                checked); entries at columns >= lens[t] are never read.
 *   lens         device int32 [T]: active counts, clamped to [0, W].
 *   bmm1_scale   score scale in natural-log units (per-tensor form: sm_scale*q_scale*k_scale).
 *   bmm2_scale   output scale (per-tensor form: k_scale).
 *   sinks        device float32 [H] natural-log sink logits, or NULL for no sink.
 *   out          device BF16 [T, H, 512] (16-byte aligned), written for every (t, h).
 *   lse          device float32 [T, H] or NULL: ln(sum_c e^{s_c} + e^{sink}) (base 2 with
 *                SMLA_LSE_LOG2); -inf for a token with no active column, whose output is +0.
 *   flags        SMLA_LSE_LOG2 | SMLA_P_ONE_TERM | SMLA_P_CHUNK_LOCAL.
 *   plan         NULL for smla_decode_plan's, else an explicit decomposition (results are
 *                bit-identical from run to run for a fixed plan).
 *   workspace    device scratch of workspace_bytes >= smla_decode_workspace_size(plan, T, H),
 *                16-byte aligned (may be NULL when that size is 0).  Zero-fill it once before
 *                its first use: its first bytes hold a status word and arrival counters that
 *                must start at zero, and every call leaves them at zero again (the partials are
 *                overwritten before they are read).  Calls that share a workspace must be
 *                stream-ordered.  With 64 heads per workgroup (plan tiles = 2) a range that
 *                merges waits for other ranges with a bounded poll (2^20 polls, each a
 *                device-memory round trip: one to two seconds in all): the last-arriver merge's last range for the others' partials, every
 *                range of a spread merge for the others' arrivals.  If the bound runs out the
 *                range adds 1 to the status word, writes NaN to the outputs and LSEs it owns and
 *                leaves the counters non-zero: a caller that finds the status word non-zero
 *                must treat those outputs as failed and zero-fill the workspace again before
 *                its next use.  (The 32-head kernel's merge never waits: every range stores
 *                first and the last to arrive merges.)
 *
 * Softmax (the attn_sparse page's recipe, module docstring): per head, chunk by chunk of 64
 * columns, the running maximum m of the base-2 scores s2 = s log2(e) rises to m' = max(m,
 * chunk maximum); everything accumulated so far (FP32 output accumulators and the FP32 sum l of
 * the unquantized P) is rescaled by alpha = 2^(m - m'); the chunk's P = 2^(s2 - m' + log2 448)
 * <= 448 is rounded to E4M3 (two terms by default, see SMLA_P_ONE_TERM) for the P.V product,
 * and its unquantized value is added to l.  Split partials merge in FP32 as smla_plan states.
 *
 * T == 0 is a no-op returning SMLA_OK after the size, flag and plan checks (the pointers are
 * not examined: empty tensors may have null data).  Errors: SMLA_EINVAL (null required
 * pointer, T < 0,
 * H <= 0 or H % 16 != 0, W < 1, bad row_bytes/qk_dim, misaligned pointer or stride,
 * split_col outside [0, W], unknown flag, non-finite scale, bad plan), SMLA_EWORKSPACE,
 * SMLA_EHIP (launch failure).
 */
smla_status sparse_mla_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                              const void *kv_a, int64_t rows_a,
                              const void *kv_b, int64_t rows_b, int32_t split_col,
                              int32_t row_bytes, int32_t qk_dim,
                              const int32_t *indices, const int32_t *lens,
                              int32_t T, int32_t H, int32_t W,
                              float bmm1_scale, float bmm2_scale, const float *sinks,
                              void *out, float *lse, uint32_t flags,
                              const smla_plan *plan, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * sparse_mla_decode_noalloc -- sparse_mla_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, results, errors and plan as sparse_mla_decode, without the workspace: the split-KV
 * workspace is a static device array of SMLA_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  No call allocates or frees anything.  Each call
 * first clears the array's status word and arrival counters with a small kernel on `stream`,
 * then runs the decode, so every call starts clean.  All calls on one GPU share that GPU's array
 * and leave their partials in it: calls that may overlap on one GPU (different streams without
 * ordering, or concurrent host threads) race and give wrong results; stream-ordered calls are
 * safe.  A problem whose workspace (smla_decode_workspace_size under the plan used) exceeds
 * SMLA_NOALLOC_SCRATCH_BYTES returns SMLA_ESCRATCH and launches nothing: the large-batch shape
 * (T = 64, H = 128, 2048 columns, default plan) needs about 34 MB.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES (48u << 20)
smla_status sparse_mla_decode_noalloc(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                                      const void *kv_a, int64_t rows_a,
                                      const void *kv_b, int64_t rows_b, int32_t split_col,
                                      int32_t row_bytes, int32_t qk_dim,
                                      const int32_t *indices, const int32_t *lens,
                                      int32_t T, int32_t H, int32_t W,
                                      float bmm1_scale, float bmm2_scale, const float *sinks,
                                      void *out, float *lse, uint32_t flags,
                                      const smla_plan *plan, hipStream_t stream);

/*
 * lse_merge -- LSE-weighted merge of S split-KV partials (dcp page, DcpValue.merge).
 *
 *   partials  device BF16 [S, T, H, D] (16-byte aligned): source s's normalized output.
 *   lse2      device float32 [S, T, H]: source s's LSE in base 2.  A source is empty unless
 *             its LSE is finite (NaN and +-inf are empty); an empty source's partial is never
 *             read.
 *   out       device BF16 [T, H, D] (16-byte aligned):
 *             sum_s (2^{lse_s - top} / sum_r 2^{lse_r - top}) x_s in FP32, one BF16 rounding;
 *             +0 where every source is empty.
 *   lse_out   device float32 [T, H] or NULL: (top + log2 sum_s 2^{lse_s - top}) in natural log
 *             (base 2 with SMLA_LSE_LOG2); -inf where every source is empty.
 *
 * S in [1, 64], D a multiple of 8.  T == 0 is a no-op (pointers not examined).  Errors: SMLA_EINVAL (null pointer,
 * bad size, misalignment, unknown flag), SMLA_EUNSUPPORTED (S > 64 or D % 8 != 0),
 * SMLA_EHIP.
 */
smla_status lse_merge(const void *partials, const float *lse2, int32_t S, int32_t T, int32_t H,
                      int32_t D, void *out, float *lse_out, uint32_t flags, hipStream_t stream);

/*
 * paged_mla_decode -- dense paged MLA decode (the dcp page, stock_decode: the FP8 cache in pages
 * addressed through a block table, the q rows of a request masked causally, caller-owned out
 * and LSE, a split-KV workspace sized before capture), on the gather and matrix skeleton of
 * sparse_mla_decode: row t = b * q_len + i (request b's i-th of q_len rows) attends over the
 * first n_t = clamp(lengths[b] - (q_len - 1 - i), 0, max_pages * page_size) keys of request b's
 * context, key k being row k % page_size of page block_table[b][k / page_size]; the score,
 * softmax recipe, split merge, outputs and flags are sparse_mla_decode's with one pool, no
 * sink and qk_dim = row_bytes = 576 (V the first 512 bytes of a row).
 *
 *   q            device, E4M3 [B * q_len, H, 576] with byte strides q_stride_t, q_stride_h
 *                (multiples of 16; 16-byte aligned).
 *   cache        device, E4M3 pages: row r of page g at cache + g * page_stride + r * 576
 *                (page_stride >= page_size * 576, a multiple of 16; 16-byte aligned).
 *   num_pages    pages in the cache: every block_table entry a row reads must be in [0,
 *                num_pages) (precondition, not checked); entries past a request's context
 *                are never read.
 *   block_table  device int32 [B, max_pages].
 *   lengths      device int32 [B]: context lengths (the q_len new rows included).
 *   out, lse     device BF16 [B * q_len, H, 512] and float32 [B * q_len, H] (or NULL).
 *   plan         NULL for smla_paged_decode_plan's, else one with tiles = 2 (64 heads per
 *                workgroup; SMLA_EUNSUPPORTED otherwise) and ranges of at most 2048 keys.
 *   workspace    as sparse_mla_decode, sized by smla_decode_workspace_size(plan, B * q_len, H).
 * Errors as sparse_mla_decode.
 */
smla_status paged_mla_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                             const void *cache, int64_t num_pages, int32_t page_size,
                             int64_t page_stride, const int32_t *block_table, int32_t max_pages,
                             const int32_t *lengths, int32_t B, int32_t q_len, int32_t H,
                             float bmm1_scale, float bmm2_scale, void *out, float *lse,
                             uint32_t flags, const smla_plan *plan, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* The plan paged_mla_decode uses when given none: 64 heads per workgroup; enough key ranges
 * over the max_pages * page_size columns to cover the compute units (at most 4, at least
 * ceil(columns / 2048), one range up to 6 chunks of 64 columns); SMLA_MERGE_SPREAD when the
 * grid, rows x head groups x ranges, fits the compute units, else SMLA_MERGE_LAST. */
smla_status smla_paged_decode_plan(int32_t B, int32_t q_len, int32_t H, int32_t max_pages,
                                   int32_t page_size, uint32_t flags, smla_plan *plan);

/*
 * mla_value -- the MLA value tail after the split merge (dcp page, DcpValue class docstring and
 * its merge method: the owner's LSE merge over the sources, then W_UV and the sigmoid gate "as
 * in MlaValue").  With S = 1 it is the value tail of sparse_mla_decode's own output (pass its
 * base-2 LSE; any finite LSE weighs 1).  For each row t < T and head h < H:
 *   latent = BF16( sum_s (2^{lse_s - top} / sum_r 2^{lse_r - top}) x_s )   (FP32 sums; sources
 *            with a non-finite LSE weigh 0 and are never read; none finite: latent = 0)
 *   out[t, 128 h + v] = BF16( BF16( sum_{k<512} latent[k] W_UV[h, k, v] ) * sigmoid(gate[t,
 *            128 h + v]) ),   W_UV in BF16, FP32 accumulation, sigmoid(g) = 1 / (1 + e^{-g}),
 * and rows whose request total totals[t / rows_per_request] is <= 0 (padded rows, whose gate
 * may be NaN) are zeros; totals == NULL makes every row live.
 *
 *   partials  device BF16 [S, T, H, 512] (16-byte aligned).
 *   lse2      device float32 [S, T, H], base 2.
 *   w_uv      device BF16: element (h, k, v) (h < H, latent k < 512, value v < 128) at
 *             w_uv + h * w_stride_h + v * w_stride_v + k: latent-contiguous, as the pages'
 *             kernel reads eight latent values per load; 16-byte aligned, strides (elements)
 *             multiples of 8.
 *   gate      device BF16 [T, H * 128].
 *   totals    device int32 [ceil(T / rows_per_request)] or NULL.
 *   out       device BF16 [T, H * 128], every element written.
 *   flags     0.
 * S in [1, 64].  T == 0 is a no-op.  Errors: SMLA_EINVAL (sizes, null pointers, alignment,
 * strides, flags), SMLA_EHIP.
 */
smla_status mla_value(const void *partials, const float *lse2, int32_t S, int32_t T, int32_t H,
                      const void *w_uv, int64_t w_stride_h, int64_t w_stride_v, const void *gate,
                      const int32_t *totals, int32_t rows_per_request, void *out, uint32_t flags,
                      hipStream_t stream);

/* A static string describing a status code (the pages raise RuntimeError or assert on bad
 * arguments; a C caller gets a status code and this text instead). */
const char *smla_strerror(smla_status status);

/* Test hook, not for production callers: bounds the 64-head kernel's split-merge wait to
 * max_polls polls (0 restores the default, 2^20) and, with unreachable = 1, makes the merging
 * range wait for one partial more than exists, so every such wait gives up after max_polls polls
 * and takes the failure path described under sparse_mla_decode while every kernel still exits
 * normally.  Process-wide; not thread-safe against concurrent calls.  SMLA_EINVAL for
 * max_polls < 0 or unreachable not in {0, 1}. */
smla_status smla_testing_set_merge_wait(int32_t max_polls, int32_t unreachable);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
