/*
 * piattn.h -- C ABI of libpiattn, a pi-Attention forward library for AMD
 * Instinct MI355X (gfx950).
 *
 * pi-Attention (Liu and Yu, arXiv 2511.10696; described on gist.science
 * "pi-Attention: Periodic Sparse Transformers for Efficient Long-Context
 * Modeling", section 2 "Methodology": "Ring-Local Attention", "pi-Skip
 * Attention" and "Dynamic Adaptive Fusion") lets query i of a sequence of
 * length n attend to the union of
 *
 *   a ring-local window   L(i) = { j : |i - j| <= k, 0 <= j < n }, with j <= i
 *                         for the causal (autoregressive) form, and
 *   periodic skip keys    S(i) = { i - m*pi : 1 <= m <= M } (plus i + m*pi in
 *                         the bidirectional form), keeping only keys inside
 *                         [0, n) and outside L(i).
 *
 * A per-query gate alpha_i = sigmoid(g_i) enters as a log-prior: log(alpha_i)
 * is added to the scaled logits of local keys and log(1 - alpha_i) to those
 * of skip keys, and one softmax runs over the union.  A row whose skip set is
 * empty gets no prior (it would be a constant shift).  Keys are never
 * wrapped around the sequence end.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The
 *     piattn_pattern struct is host memory, read during the call only.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  The library keeps no
 *     state besides a thread-local error string and allocates no memory:
 *     scratch space is a caller-provided workspace (see the *_workspace_bytes
 *     queries).
 *   - Every argument is validated before anything is launched.  A non-zero
 *     status is returned on error and piattn_last_error() describes it.
 *     Nothing aborts and nothing throws across the ABI.
 *   - Element strides are given per tensor as {sequence, head, token}, in
 *     elements; the head dimension d is always contiguous.
 */
#ifndef PIATTN_H
#define PIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and the output.  Gate logits are always fp32.
 * The two range enumerators only widen the type's range of values to every
 * int32, so that any value a caller passes is a value of the type; the
 * entry points accept PIATTN_F32 and PIATTN_BF16 and reject the rest with
 * PIATTN_EINVAL. */
typedef enum {
    PIATTN_F32 = 0,
    PIATTN_BF16 = 1,
    PIATTN_DTYPE_RANGE_LO_ = -0x7fffffff - 1,
    PIATTN_DTYPE_RANGE_HI_ = 0x7fffffff
} piattn_dtype;

/* Status codes. */
enum {
    PIATTN_OK = 0,
    PIATTN_EINVAL = 1,       /* bad pointer, size, stride, alignment or pattern */
    PIATTN_EUNSUPPORTED = 2, /* valid request the library does not implement */
    PIATTN_EWORKSPACE = 3,   /* workspace missing or too small */
    PIATTN_EHIP = 4          /* the HIP runtime reported a launch error */
};

/*
 * The sparsity pattern (the pages' n, k, pi; M and the gate form as stated
 * above).
 *   window_k      k >= 0: keys i-k..i (causal) or i-k..i+k (bidirectional)
 *   period_pi     pi >= 1: skip stride
 *   num_skips_M   M >= 0: skips per direction
 *   bidirectional 0 = causal, 1 = two-sided window and skips
 *   scale         logit scale; <= 0 selects 1/sqrt(d)
 *   num_levels    0..PIATTN_MAX_LEVELS: extra skip levels (a skip schedule,
 *                 the hierarchical schedules the Dutch gist.science summary
 *                 names as future work, section 5 "Betekenis en Conclusie");
 *                 level r adds the skips i -/+ m*level_pi[r], 1 <= m <=
 *                 level_M[r].  The skip set is the union over (period_pi,
 *                 num_skips_M) and the extra levels, each key once, every
 *                 skip key with the log(1 - alpha) prior.  With extra levels
 *                 the distinct skip distances beyond the window must be
 *                 multiples m*g, m < 128, of g = gcd of the periods of the
 *                 levels with M > 0 (else PIATTN_EUNSUPPORTED).
 * A zero-initialised tail (num_levels = 0) is the single-period pattern.
 */
#define PIATTN_MAX_LEVELS 7
typedef struct {
    int32_t window_k;
    int32_t period_pi;
    int32_t num_skips_M;
    int32_t bidirectional;
    float scale;
    int32_t num_levels;
    int32_t level_pi[PIATTN_MAX_LEVELS];
    int32_t level_M[PIATTN_MAX_LEVELS];
} piattn_pattern;

/*
 * piattn_fwd -- prefill: every query row of every (sequence, head).
 *
 * Dense mode (cu_seqlens == NULL): B sequences of n tokens each.  Element
 * (b, h, t, c) of q, k, v, out lives at
 *     base + b*s[0] + h*s[1] + t*s[2] + c
 * with s = strides[0] (q), strides[1] (k), strides[2] (v), strides[3] (out).
 * Gate logit (b, h, t) lives at gate_logits + b*s[0] + h*s[1] + t*s[2] with
 * s = strides[4]; lse_out (optional, may be NULL) uses the same addressing
 * and receives the natural-log normaliser log(sum_j exp(logit_j)) of each
 * row, logits including the prior.
 *
 * Varlen mode (cu_seqlens != NULL): B packed sequences; sequence b occupies
 * tokens [cu_seqlens[b], cu_seqlens[b+1]) of one packed token axis (device
 * int32 array of B+1 non-decreasing offsets starting at 0).  The sequence
 * stride s[0] is ignored and t is the packed token index.  n must be >= the
 * longest sequence: the grid covers n rows per sequence and the library reads
 * cu_seqlens on the device only, so it cannot report a longer sequence; such
 * a sequence is cut at n rows (its later rows are neither read as keys nor
 * written), and nothing is indexed beyond n rows of any buffer.  No
 * attention crosses a sequence boundary.
 *
 * Requirements: B, H, n >= 1; d in {32, 64, 128}; for PIATTN_BF16 the q, k,
 * v, out pointers are 16-byte aligned and their strides multiples of 8
 * elements; for PIATTN_F32, 16-byte aligned and multiples of 4 elements.
 * The output must not alias an input.  Indices must fit in int64.
 *
 * workspace: device scratch of at least piattn_fwd_workspace_bytes(dtype, B,
 * H, n, d, pattern) bytes, 256-byte aligned; may be NULL when that is 0.
 * The bf16 d = 64 / 128 path splits the work into a skip pass and a window
 * pass and hands one (log-sum-exp, exponent) float pair per row from the
 * first to the second through it.  Calls that share a workspace must be
 * ordered (the same stream, or synchronised); its contents are scratch
 * before and after a call.
 * Returns PIATTN_OK, PIATTN_EINVAL, PIATTN_EUNSUPPORTED, PIATTN_EWORKSPACE
 * (workspace NULL or too small) or PIATTN_EHIP.
 */
int piattn_fwd(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d,
               const void *q, const void *k, const void *v,
               const float *gate_logits, void *out, float *lse_out,
               const int64_t strides[5][3], const int32_t *cu_seqlens,
               const piattn_pattern *pattern, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * piattn_fwd_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): piattn_fwd with the same arguments and results, whose
 * workspace is a library-held device array of PIATTN_NOALLOC_SCRATCH_BYTES
 * instead of a caller buffer.  The caller still passes the inputs and the
 * outputs.  Nothing is allocated by the call: each GPU the library runs on
 * holds its own copy of the array, zero when first used, until the process
 * ends; its address is looked up once per device.  A call whose workspace
 * need (piattn_fwd_workspace_bytes) exceeds the array returns
 * PIATTN_EWORKSPACE.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that may overlap on one GPU (on
 * different streams without ordering, or from several threads) race and
 * must not be issued.  Returns what piattn_fwd returns.
 */
#define PIATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int piattn_fwd_noalloc(piattn_dtype dtype, int32_t B, int32_t H, int32_t n,
                       int32_t d, const void *q, const void *k, const void *v,
                       const float *gate_logits, void *out, float *lse_out,
                       const int64_t strides[5][3], const int32_t *cu_seqlens,
                       const piattn_pattern *pattern, void *stream);

/*
 * Workspace piattn_fwd needs for these sizes and pattern: for PIATTN_BF16
 * with d in {64, 128} when the pattern has skip keys (num_skips_M >
 * window_k / period_pi), 8*B*H*n bytes rounded up to a multiple of 256, plus
 * 128*(9 + B*H*ceil(ceil(n/pi)/16)) bytes of schedule counters (one 128-byte
 * line each; pi: the period, or the periods' gcd of a skip schedule); else
 * 0.  0 also for invalid arguments (piattn_fwd reports those).
 */
size_t piattn_fwd_workspace_bytes(piattn_dtype dtype, int32_t B, int32_t H,
                                  int32_t n, int32_t d,
                                  const piattn_pattern *pattern);

/*
 * piattn_bwd -- backward of piattn_fwd (the pages train pi-Attention
 * models: gist.science section 4 "Experimental Results", item
 * "Computational Efficiency", training speed; its section 2 "Execution &
 * Scheduling" overlaps micro-batches in training).  Given the forward's
 * inputs, its output `out`, optionally its log-sum-exp `lse`, and the
 * gradient `dout` of a loss with respect to out, writes the gradients with
 * respect to q, k, v (dq, dk, dv; element type of q) and the gate logits
 * (dgate, fp32).  Per row i with keys j (one softmax P_ij over L(i) u S(i)):
 * dS_ij = P_ij (<dout_i, v_j> - <dout_i, out_i>),
 * dq_i = scale sum_j dS_ij k_j, dk_j = scale sum_i dS_ij q_i,
 * dv_j = sum_i P_ij dout_i, dgate_i = (1 - alpha_i) sum_{j in L} dS_ij -
 * alpha_i sum_{j in S} dS_ij (0 on rows without skip keys).
 *
 * lse: the forward's lse_out (natural log, addressed like the gate logits),
 * or NULL.  Given lse, PIATTN_BF16 with d in {64, 128} runs on MFMA (P from
 * the saved lse; a skip pass then a window pass, the skip part of dq, dk, dv
 * held as bf16 in the gradient rows in between).  Otherwise, or with NULL,
 * each row's softmax is recomputed in fp32 on the gather path.
 *
 * Shapes, modes and requirements as for piattn_fwd; dq, dk, dv use the
 * strides of q, k, v (strides[0..2]), dout those of out (strides[3]) and
 * dgate those of the gate logits (strides[4]).  No gradient may alias an
 * input or another gradient.  workspace: device scratch of at least
 * piattn_bwd_workspace_bytes(B, H, n) bytes (16 per row), 256-byte aligned.
 * Returns PIATTN_OK, PIATTN_EINVAL, PIATTN_EUNSUPPORTED, PIATTN_EWORKSPACE
 * or PIATTN_EHIP.
 */
int piattn_bwd(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d,
               const void *q, const void *k, const void *v,
               const float *gate_logits, const void *out, const float *lse,
               const void *dout, void *dq, void *dk, void *dv, float *dgate,
               const int64_t strides[5][3], const int32_t *cu_seqlens,
               const piattn_pattern *pattern, void *workspace,
               size_t workspace_bytes, void *stream);

/* Workspace bytes piattn_bwd needs: 16 * B * H * n (0 for invalid sizes). */
size_t piattn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t n);

/*
 * The linear maps around the attention.  The pages give the gate as a
 * learnable shallow MLP of the input (gist.science section 2 "Methodology",
 * item "Dynamic Adaptive Fusion") and end with a fusion-and-projection
 * stage (section 2 "Execution & Scheduling", "Streaming Stages"); the
 * plainest form is taken: one linear layer per head for the gate logit and
 * the usual output projection of the concatenated heads.
 *
 * piattn_gate_logits -- g[b, h, i] = <x[b, i, :], w[h, :]> + bias[h], fp32,
 * written in the prefill's gate layout.
 *   x [B, n, Dm]     element (b, i, c) at x + b*x_strides[0] + i*x_strides[1] + c
 *   w [H, Dm]        row-major, contiguous
 *   bias [H]         fp32, or NULL
 *   g                element (b, h, i) at g + b*s[0] + h*s[1] + i*s[2], s = g_strides
 * PIATTN_BF16 (x, w) runs on MFMA and needs Dm % 32 == 0, H <= 32, x and w
 * 16-byte aligned with strides multiples of 8 (else EUNSUPPORTED / EINVAL);
 * PIATTN_F32 runs a plain kernel.  Returns PIATTN_OK, EINVAL, EUNSUPPORTED
 * or EHIP.
 */
int piattn_gate_logits(piattn_dtype dtype, int32_t B, int32_t n, int32_t Dm, int32_t H,
                       const void *x, const int64_t x_strides[2], const void *w,
                       const float *bias, float *g, const int64_t g_strides[3],
                       void *stream);

/*
 * piattn_out_proj -- y[b, i, :] = sum_{h, c} o[b, h, i, c] w[:, h*d + c] + bias,
 * the output projection of the concatenated heads, read straight from the
 * attention's output layout (no copy).
 *   o [B, H, n, d]   element (b, h, i, c) at o + b*s[0] + h*s[1] + i*s[2] + c, s = o_strides
 *   w [Dout, H*d]    row r at w + r*ldw (ldw >= H*d), contiguous columns
 *   bias [Dout]      fp32, or NULL
 *   y [B, n, Dout]   element (b, i, c) at y + b*y_strides[0] + i*y_strides[1] + c
 * Element type of o, w, y: dtype.  PIATTN_BF16 with d % 32 == 0 runs an MFMA
 * GEMM (fp32 accumulation, bf16 round-to-nearest-even store); other shapes
 * and PIATTN_F32 a plain kernel.  bf16 needs 16-byte alignment and strides
 * (and ldw) that are multiples of 8 elements.  y must not alias o or w.
 * Returns PIATTN_OK, EINVAL or EHIP.
 */
int piattn_out_proj(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d,
                    const void *o, const int64_t o_strides[3], int32_t Dout, const void *w,
                    int64_t ldw, const float *bias, void *y, const int64_t y_strides[2],
                    void *stream);

/*
 * piattn_decode -- one new query per sequence against its KV cache (the
 * pages' inference mode, gist.science section 2 "Execution & Scheduling",
 * item "Inference").  The query of sequence s sits at position
 * cache_lens[s] - 1: its own key and value are already in the cache, and it
 * attends causally over the window and skips of that position.
 *
 *   q [S, H, d]               element (s, h, c) at q + s*s0 + h*s1 + c,
 *                             {s0, s1, -} = strides[0]
 *   k_cache, v_cache          element (s, h, t, c) at base + s*s0 + h*s1 + t*s2 + c,
 *                             strides[1], strides[2]; t < cache_capacity
 *   cache_lens [S]            device int32; a row whose length is outside
 *                             [1, cache_capacity] is written as NaN
 *   gate_logits [S, H]        fp32, strides[4] (token stride ignored)
 *   out [S, H, d]             strides[3] (token stride ignored)
 *   pattern                   must be causal (bidirectional == 0)
 *   num_splits                key-range splits per (sequence, head); 0 = auto
 *   workspace                 device scratch of at least
 *                             piattn_decode_workspace_bytes(S, H, d, num_splits,
 *                             pattern)
 *                             bytes, 256-byte aligned (unused, may be NULL, when
 *                             that size is 0)
 * Alignment rules as for piattn_fwd.  Calls that share a workspace must be
 * ordered on one stream.
 */
int piattn_decode(piattn_dtype dtype, int32_t S, int32_t H, int32_t d,
                  const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *cache_lens, int32_t cache_capacity,
                  const float *gate_logits, void *out,
                  const int64_t strides[5][3], const piattn_pattern *pattern,
                  int32_t num_splits, void *workspace, size_t workspace_bytes,
                  void *stream);

/* Workspace bytes piattn_decode needs for this shape and split count
 * (num_splits 0 = the automatic choice for `pattern`).  0 means no workspace
 * is needed; 0 is also returned for invalid arguments. */
size_t piattn_decode_workspace_bytes(int32_t S, int32_t H, int32_t d,
                                     int32_t num_splits,
                                     const piattn_pattern *pattern);

/* Number of splits piattn_decode uses for num_splits = 0 on this shape. */
int32_t piattn_decode_auto_splits(int32_t S, int32_t H, int32_t d,
                                  const piattn_pattern *pattern);

/*
 * Rolling KV cache for decode.  The pages note that at inference the cache
 * is updated in constant time because a new token only touches positions
 * modulo pi (gist.science section 2 "Execution & Scheduling", item
 * "Inference"), and a sliding-window model keeps its keys and values in a
 * buffer of w rows, position i in row i mod w, overwriting the oldest
 * (Ultralytics glossary "Sliding Window Attention", section "Wie das
 * Fenster mit der Tiefe wächst").  Here the newest position i attends to
 * i-k .. i and i - m*pi, m <= M, so a cache of W = max(k, M*pi) + 1 rows
 * (k + 1 when the pattern has no skip keys outside the window), position j
 * in row j mod W, holds every key it needs, whatever the sequence length.
 */

/* W for this pattern (-1 for an invalid pattern or W >= 2^30). */
int32_t piattn_rolling_slots(const piattn_pattern *pattern);

/*
 * Append one token per sequence: for every (s, h), the key and value rows
 * k_new[s, h, :] and v_new[s, h, :] are written to row positions[s] mod
 * cache_slots of k_cache[s, h] and v_cache[s, h].  positions is a device
 * int32 array [S]; a negative entry leaves that sequence's rows alone.
 * strides[0], strides[1]: {s0, s1, -} of k_new, v_new ([S, H, d]);
 * strides[2], strides[3]: {s0, s1, row} of the caches ([S, H, cache_slots, d]).
 * Pointers need the element alignment only.  Returns PIATTN_OK,
 * PIATTN_EINVAL, PIATTN_EUNSUPPORTED (d) or PIATTN_EHIP.
 */
int piattn_cache_append(piattn_dtype dtype, int32_t S, int32_t H, int32_t d,
                        const void *k_new, const void *v_new, void *k_cache,
                        void *v_cache, const int32_t *positions,
                        int32_t cache_slots, const int64_t strides[4][3],
                        void *stream);

/*
 * piattn_decode over a rolling cache: arguments as for piattn_decode, with
 * cache_slots rows per (sequence, head) holding position j in row j mod
 * cache_slots.  cache_lens[s] (the number of tokens so far; the query sits
 * at position cache_lens[s] - 1, already appended) may exceed cache_slots;
 * a length below 1 gives a NaN row, and lengths must stay below 2^30.
 * cache_slots must be at least piattn_rolling_slots(pattern) (else
 * PIATTN_EINVAL).  The result equals piattn_decode on a linear cache that
 * holds the same positions.
 */
int piattn_decode_rolling(piattn_dtype dtype, int32_t S, int32_t H, int32_t d,
                          const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *cache_lens, int32_t cache_slots,
                          const float *gate_logits, void *out,
                          const int64_t strides[5][3], const piattn_pattern *pattern,
                          int32_t num_splits, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * piattn_neighbors -- debug dump of the neighbour lists that the compute
 * kernels enumerate, for queries q_begin .. q_begin+q_count-1 of a sequence
 * of length n.  Row r of idx [q_count, cap] (device int32) receives the keys
 * in ascending order, padded with -1; kind [q_count, cap] (device int8)
 * receives 1 for a local key, 2 for a skip key, 0 for padding; count
 * [q_count] (device int32) the list length.  cap must be at least
 * piattn_neighbors_cap(pattern).
 */
int piattn_neighbors(int32_t n, const piattn_pattern *pattern, int32_t q_begin,
                     int32_t q_count, int32_t cap, int32_t *idx, int8_t *kind,
                     int32_t *count, void *stream);

/* Longest possible list: (k+1)+M causal, (2k+1)+2M bidirectional; -1 if the
 * pattern is invalid. */
int32_t piattn_neighbors_cap(const piattn_pattern *pattern);

/*
 * Testing and measurement hook (not for production dispatch): force the
 * kernel that piattn_fwd and piattn_bwd run for every later call in this
 * process.  PIATTN_KERNEL_AUTO (0) restores the automatic choice (the first
 * kernel that can take a call).  A forced kernel that cannot take a call
 * makes that call return PIATTN_EUNSUPPORTED.  The setting is process-wide
 * and read once per call; change it only while no other thread calls into
 * the library.  Returns PIATTN_OK, or PIATTN_EINVAL for an unknown id.
 */
enum {
    PIATTN_KERNEL_AUTO = 0,
    PIATTN_FWD_SPLIT = 1,   /* skip pass + window pass (bf16, d 64 / 128) */
    PIATTN_FWD_RESID = 2,   /* residue-tiled single kernel (bf16, d 64) */
    PIATTN_FWD_GATHER = 3,  /* one wave per row (any dtype and d) */
    PIATTN_FWD_F32MFMA = 4, /* fp32 on fp32 MFMA, 16 query rows per wave (fp32, d 32 / 64 / 128) */
    PIATTN_FWD_LAST = PIATTN_FWD_F32MFMA,
    PIATTN_BWD_BAND = 1,    /* MFMA band kernels (bf16, d 64 / 128, lse given) */
    PIATTN_BWD_GATHER = 2   /* gather kernels (any dtype and d) */
};
int piattn_debug_force_kernels(int32_t fwd_kernel, int32_t bwd_kernel);

/* Description of the last error on this thread ("" if none). */
const char *piattn_last_error(void);

/* Library version string. */
const char *piattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PIATTN_H */
