/*
 * hs2.h — C ABI of libhs2.so: the HySparse2 Cross-Decoder attention hot path
 * (one full-attention layer that also scores every key, a token-level top-k
 * with a forced recent window, and several sparse-attention layers that reuse
 * the same KV cache and the same index list) for AMD Instinct MI355X (gfx950).
 *
 * Where the method comes from
 *   - KV Reuse: the KV cache and the token-selection result of one full
 *     attention layer are handed to the sparse layers that follow it
 *     (news page "两天两连更：小米提前亮出V3底牌", section
 *     "两级KV共享：让模型少跑一半").
 *   - Token-level selection, a fixed window of the most recent tokens plus a
 *     chosen set of older tokens, one shared cache for both (same page,
 *     section "Token级选择：精准定位大海里的那根针"; the experiments there keep
 *     128 recent tokens and choose 1024 older ones).
 *   - The selection comes from the full layer's own attention, with no
 *     separately trained indexer (video page "小米 MiMo-V3 HySparse2
 *     架构：读长文省一半", section "HySparse2 的解法：两派都用，还改了流程").
 *   The pages do not say how the query heads of a GQA group combine into one
 *   importance per key; this library uses the largest softmax probability any
 *   head of the group gives the key, ties going to the lower key index, one
 *   selection per (batch, query token, KV head).
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major, in device memory of the current HIP
 *     device, allocated and owned by the caller; the library never allocates,
 *     frees or synchronises on these calls and keeps no global mutable state
 *     (the last HIP error code is thread-local).  Outputs must not overlap
 *     inputs or each other.
 *   - bf16 tensors hold raw bfloat16 bit patterns (hs2_bf16).
 *   - Query token t of a chunk of T tokens sits at position P_t = S - T + t
 *     and sees keys 0..P_t (its own key included).  Decode is T = 1.
 *   - Layouts:  q, out            [B][T][Hq][D]
 *               q_sparse, out_sp  [N][B][T][Hq][D]
 *               k, v (KV cache)   [B][Hkv][Sc][D]  token-major per KV head, Sc =
 *                                                 kv_capacity (ctx_len when 0); rows
 *                                                 S..Sc-1 are not read
 *               lse               [B][T][Hq]        natural log, float32
 *               scores            [B][T][Hkv][S]    float32, 0 past P_t
 *               idx               [B][T][Hkv][k+w]  int32, ascending, -1 past n_sel
 *               n_sel             [B][T][Hkv]       int32
 *   - `ws` is a caller-owned device workspace of at least
 *     hs2_workspace_bytes(shape, n_layers) bytes, 256-byte aligned; its
 *     contents need no initialisation and are scratch after the call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; results are ready when the stream reaches that point.
 *   - Errors: argument and shape errors are detected on the host before
 *     anything is enqueued (HS2_ERR_INVALID_ARG, HS2_ERR_UNSUPPORTED,
 *     HS2_ERR_WORKSPACE).  A failed launch returns HS2_ERR_HIP and keeps the
 *     hipError_t in hs2_last_hip_error().  Faults inside kernels surface at the
 *     caller's next synchronisation, as HIP reports them.
 *   - v1 supports head_dim = 128 and Hq = 8 * Hkv exactly, S < 2^31,
 *     top_k + window <= 4096.
 */
#ifndef HS2_H_
#define HS2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t hs2_bf16; /* raw bfloat16 bits */

typedef struct hs2_shape {
  int64_t ctx_len;    /* S: keys 0..S-1, including the query tokens' own keys */
  double scale;       /* softmax scale, normally 1/sqrt(D); kept in double because the
                         float64 re-ranking near the k-th threshold needs it exactly */
  int32_t batch;      /* B */
  int32_t n_q_tokens; /* T: 1 = decode; > 1 = a prefill chunk (the last T positions) */
  int32_t n_q_heads;  /* Hq */
  int32_t n_kv_heads; /* Hkv; the GQA group size is G = Hq / Hkv */
  int32_t head_dim;   /* D */
  int32_t top_k;      /* k: older tokens chosen per row (1024 in the pages' experiments) */
  int32_t window;     /* w: most recent tokens always kept (128 in the pages' experiments) */
  int32_t select_block;/* 0: token-level selection (this method).  A power of two in
                         16..256: the previous generation's block-level variant, for
                         comparison: the older tokens [0, P_t-w+1) are cut into aligned
                         blocks of this many tokens (the last one ends at P_t-w+1), a
                         block's importance is the largest importance of its tokens, and
                         the top_k / select_block best blocks are kept, ties to the lower
                         block; the window is kept as before.  Needs top_k to be a
                         multiple of it and ceil(ctx_len / select_block) <= 16384.  A
                         row's last block ends at the window, so a row that takes it holds
                         fewer than top_k older tokens. */
  int64_t kv_capacity;/* token rows per KV head in k and v, i.e. the cache's row pitch:
                         row j of head (b, g) starts at element ((b*Hkv + g)*kv_capacity + j)*D.
                         0 means ctx_len; otherwise it must be >= ctx_len.  Rows ctx_len ..
                         kv_capacity-1 are never read, so a cache allocated once for its
                         final length serves every step as it grows (see hs2_kv_bridge). */
  int32_t decode_splits;/* 0: the library's plan.  Otherwise the number of context splits
                         per row of the decode full layer (clamped to 1 .. min(1024,
                         ceil(ctx_len / 128))), e.g. to check that the results do not
                         depend on the plan.  Ignored for a prefill chunk. */
  int32_t decode_select;/* 0: the library's plan.  1: the decode selection from the full
                         layer's 16-key subtile bounds (re-reading the K rows of the
                         candidates only); 2: from every key's importance (one pass over
                         K, then the same ranking as a prefill chunk's rows).  The plan
                         takes 2 where all of K is small (short contexts).  Both give the
                         same selection; e.g. to test both.  Ignored for a prefill chunk;
                         other values give HS2_ERR_INVALID_ARG. */
} hs2_shape;          /* 64 bytes, no padding */

enum {
  HS2_OK = 0,
  HS2_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad workspace alignment */
  HS2_ERR_UNSUPPORTED = -2, /* a valid shape this build does not implement */
  HS2_ERR_WORKSPACE = -3,   /* ws_bytes smaller than hs2_workspace_bytes() */
  HS2_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  HS2_ERR_SCRATCH = -5      /* the shape needs more than the static scratch (see
                               hs2_cross_decoder_step_static) */
};

/* Bytes of workspace any call below needs for this shape and number of sparse
 * layers (the maximum over the calls, so one buffer serves all of them).
 * Returns 0 if the shape is invalid or unsupported. */
size_t hs2_workspace_bytes(const hs2_shape* shape, int32_t n_sparse_layers);

/* Full attention over the shared cache, with per-key importance.
 * For every (b, t, KV head g) and query head h of the group:
 *   s_h[j] = scale * <q_h, k_j> for j <= P_t,  out_h = softmax(s_h) . V,
 *   lse_h  = log sum_j exp(s_h[j]),  scores[j] = max_h softmax(s_h)[j].
 * q [B][T][Hq][D], k/v [B][Hkv][Sc][D] in; out [B][T][Hq][D] out.
 * lse (nullable) [B][T][Hq]; scores (nullable) [B][T][Hkv][S] (0 past P_t).
 * This is the group's full-attention layer: news page, section
 * "两级KV共享：让模型少跑一半" (KV Reuse), and video page, section
 * "HySparse2 的解法：两派都用，还改了流程" (selection from the attention). */
int hs2_full_attn_scores(const hs2_shape* shape, const hs2_bf16* q, const hs2_bf16* k,
                         const hs2_bf16* v, hs2_bf16* out, float* lse, float* scores,
                         void* ws, size_t ws_bytes, void* stream);

/* Token-level selection from given scores [B][T][Hkv][S] (float32, compared
 * exactly as given).  For each row: keep the window [max(0, P_t-w+1), P_t];
 * from the older keys [0, P_t-w+1) keep the top_k with the largest score,
 * ties to the lower index (all of them if fewer than top_k).  Writes idx
 * [B][T][Hkv][k+w] ascending (-1 past n_sel) and n_sel [B][T][Hkv].
 * News page, section "Token级选择：精准定位大海里的那根针". */
int hs2_topk_select(const hs2_shape* shape, const float* scores, int32_t* idx, int32_t* n_sel,
                    void* ws, size_t ws_bytes, void* stream);

/* Sparse attention of n_layers layers that reuse one KV cache and one index
 * list per row: for layer n, out^(n)_h = softmax_i(scale * <q^(n)_h, k_i>) . V_i
 * over i in idx[b][t][g][0..n_sel).  q [N][B][T][Hq][D], out [N][B][T][Hq][D];
 * idx / n_sel as written by hs2_topk_select (entries must be in [0, P_t];
 * an entry outside [0, S) is clamped into it, so a malformed list gives wrong
 * numbers for its row but never an out-of-bounds read, and every entry
 * outside [0, P_t] is counted in the workspace: HS2_WS_INDEX_CHECK).
 * Rows with n_sel = 0 get zero outputs.  News page, section
 * "两级KV共享：让模型少跑一半" (the sparse layers reuse the cache and the
 * selection). */
int hs2_sparse_attn(const hs2_shape* shape, int32_t n_layers, const hs2_bf16* q,
                    const hs2_bf16* k, const hs2_bf16* v, const int32_t* idx,
                    const int32_t* n_sel, hs2_bf16* out, void* ws, size_t ws_bytes,
                    void* stream);

/* The previous generation's sparse layer, for comparison: a separate sliding-
 * window branch with the layer's own local K/V, next to attention over the
 * selected older tokens of the shared cache (news page, section
 * "Token级选择：精准定位大海里的那根针": HySparse2 drops this branch and its
 * extra projections and local cache, and forces the window into the shared
 * selection instead).  For layer n and head h of row (b, t, g):
 *   out = softmax(scale q k_sel) . V_sel  +  softmax(scale q k_loc_win) . v_loc_win
 * where sel = the entries of idx below P_t - w + 1 (the window entries that the
 * selection appends to the list are not read), and win = the local rows of
 * positions [max(0, P_t - w + 1), P_t].  Each branch has its own softmax; the
 * pages give no gate, so the two outputs are added.  An empty branch adds 0.
 *   k_loc, v_loc  [N][B][Hkv][Lc][D] bf16, Lc = min(S, T + w - 1): each layer's
 *                 local cache of the positions S - Lc .. S - 1 (row i holds
 *                 position S - Lc + i); with no rows (w = 0 in decode) they
 *                 may be NULL
 * Other arguments as in hs2_sparse_attn (k, v read with the kv_capacity pitch). */
int hs2_sparse_attn_swa(const hs2_shape* shape, int32_t n_layers, const hs2_bf16* q,
                        const hs2_bf16* k, const hs2_bf16* v, const int32_t* idx,
                        const int32_t* n_sel, const hs2_bf16* k_loc, const hs2_bf16* v_loc,
                        hs2_bf16* out, void* ws, size_t ws_bytes, void* stream);

/* One Cross-Decoder group step: full attention with importance, selection,
 * then n_sparse_layers sparse layers — the same results as the three calls
 * above in sequence, except that the selection here ranks keys by importance
 * computed in float64 from exact bf16 products (so that keys are ordered by
 * their exact importance, not by its float32 rounding).  scores and lse are
 * nullable.  q_sparse / out_sparse may be NULL when n_sparse_layers = 0.
 * Both decode (n_q_tokens = 1) and a prefill chunk (n_q_tokens > 1, one
 * selection per query token) are supported. */
int hs2_cross_decoder_step(const hs2_shape* shape, int32_t n_sparse_layers,
                           const hs2_bf16* q_full, const hs2_bf16* q_sparse,
                           const hs2_bf16* k, const hs2_bf16* v, hs2_bf16* out_full,
                           hs2_bf16* out_sparse, int32_t* idx, int32_t* n_sel, float* lse,
                           float* scores, void* ws, size_t ws_bytes, void* stream);

/* The step above for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results, minus the workspace, which here is a buffer
 * of HS2_STATIC_SCRATCH_BYTES that the library holds in device memory on
 * every GPU it runs on, until the process ends.  The call allocates nothing.
 * Its first call on a device looks up that device's buffer (with the device
 * current, as for every call), so make one call before a graph capture.
 *   - Shapes whose hs2_workspace_bytes exceeds HS2_STATIC_SCRATCH_BYTES get
 *     HS2_ERR_SCRATCH, before anything is enqueued (the decode workloads up to
 *     1M keys over B * n_kv_heads = 4 rows, or 256K keys over 16 rows, fit).
 *   - Every call on a GPU shares that GPU's buffer, whose contents are those
 *     of the last call: calls that may overlap on one GPU (other streams,
 *     other threads) race and must be ordered by the caller.
 *   - hs2_workspace_region's regions are not reachable for this buffer.
 * Other errors as hs2_cross_decoder_step. */
#define HS2_STATIC_SCRATCH_BYTES ((size_t)96 << 20)
int hs2_cross_decoder_step_static(const hs2_shape* shape, int32_t n_sparse_layers,
                                  const hs2_bf16* q_full, const hs2_bf16* q_sparse,
                                  const hs2_bf16* k, const hs2_bf16* v, hs2_bf16* out_full,
                                  hs2_bf16* out_sparse, int32_t* idx, int32_t* n_sel,
                                  float* lse, float* scores, void* stream);

/* The step above, with HIP events recorded on `stream` between its phases,
 * for measurement: phase_ms[0] = full-attention split kernel, [1] = combine,
 * [2] = selection (all its kernels), [3] = sparse layers (kernel + combine).
 * Runs `iters` steps back to back, synchronises the stream and returns the
 * average milliseconds of each phase.  Not for the serving loop. */
int hs2_cross_decoder_step_timed(const hs2_shape* shape, int32_t n_sparse_layers,
                                 const hs2_bf16* q_full, const hs2_bf16* q_sparse,
                                 const hs2_bf16* k, const hs2_bf16* v, hs2_bf16* out_full,
                                 hs2_bf16* out_sparse, int32_t* idx, int32_t* n_sel,
                                 void* ws, size_t ws_bytes, void* stream, int32_t iters,
                                 float* phase_ms /* [4] */);

/* ---- KV Bridging: the cache rows themselves -------------------------------
 * The Cross-Decoder's full-attention layer builds its K and V from the
 * Self-Decoder's hidden states (news page, section
 * "两级KV共享：让模型少跑一半", item "KV Bridging").  The page gives no formula;
 * this call reads it as a plain linear projection per KV head (no bias, no
 * normalisation or position transform inside it):
 *   K[b][g][pos0 + t][d] = sum_m w_kv[0][g][d][m] * hidden[b][t][m]
 *   V[b][g][pos0 + t][d] = sum_m w_kv[1][g][d][m] * hidden[b][t][m]
 * accumulated in float32 and rounded to bf16 (nearest even).
 *   hidden  [B][n][d_model]        bf16, the new tokens' hidden states
 *   w_kv    [2][Hkv][D][d_model]   bf16, one weight row per output feature
 *   k, v    [B][Hkv][kv_capacity][D] bf16 caches (the layout every call above
 *           reads with kv_capacity as the row pitch); only rows pos0 .. pos0+n-1
 *           of each head are written.
 * n = 1 with pos0 = S - 1 is the decode-time append of the token that the
 * next hs2_cross_decoder_step (ctx_len = S, same kv_capacity) attends from.
 * No workspace.  Errors: null pointers, non-positive sizes, reserved != 0 or
 * pos0 + n > kv_capacity give HS2_ERR_INVALID_ARG; head_dim != 128, a
 * d_model that is not a multiple of 64 or above 2^20, more than 4096 KV heads
 * or B * n >= 2^31 give HS2_ERR_UNSUPPORTED.  k and v must not overlap hidden
 * or w_kv. */
typedef struct hs2_bridge_shape {
  int64_t kv_capacity; /* token rows per KV head of k and v */
  int64_t pos0;        /* cache position of the first new token */
  int32_t batch;       /* B */
  int32_t n_tokens;    /* n: new tokens per batch entry */
  int32_t d_model;     /* hidden size of the Self-Decoder output */
  int32_t n_kv_heads;  /* Hkv */
  int32_t head_dim;    /* D */
  int32_t reserved;    /* must be 0 */
} hs2_bridge_shape;    /* 40 bytes, no padding */

int hs2_kv_bridge(const hs2_bridge_shape* shape, const hs2_bf16* hidden, const hs2_bf16* w_kv,
                  hs2_bf16* k, hs2_bf16* v, void* stream);

/* ---- Introspection (tests and diagnostics) ---------------------------------
 * Where a named piece of the state that a step leaves in its workspace sits,
 * for this shape and number of sparse layers: *offset (bytes from the start of
 * ws) and *bytes.  The regions:
 *   HS2_WS_LSE2  float64 [B][T][Hq]: each query head's base-2 log-normaliser,
 *                log2 sum_j 2^(c2 s_j) with c2 = scale * log2(e) (the natural-log
 *                lse divided by ln 2), as the selection ranks keys with it.
 *                Valid after hs2_cross_decoder_step, and in decode after
 *                hs2_full_attn_scores.
 *   HS2_WS_REFINE uint32 [B*T*Hkv rows][4]: the refinement of that normaliser
 *                over the keys that carry weight (see hs2_cross_decoder_step).
 *                Decode with the subtile selection (and hs2_full_attn_scores):
 *                [0] dominant 16-key subtiles summed again, [1] subtiles whose
 *                recomputed float32 maximum differed from the full layer's
 *                (expected 0), [2] 0.  A prefill chunk, and decode with the
 *                dense selection (shape.decode_select): [0] dominant keys
 *                summed again, [1] heads whose normaliser moved by more than
 *                the selection's error bound allows (expected 0), [2] dominant
 *                keys beyond the per-row list capacity (not summed again;
 *                expected 0).  [3]: the token-level per-row selection (a
 *                prefill chunk, or decode with the dense selection), the
 *                older keys its pass listed as within reach of the band
 *                (above 8192 the band is found by a second read of the row);
 *                otherwise 0.  Valid after hs2_cross_decoder_step (and, in
 *                decode, hs2_full_attn_scores).
 *   HS2_WS_INDEX_CHECK uint32 [B*T*Hkv rows][n_parts]: the sparse layers' index
 *                check.  Summed over a row's n_parts (bytes / (rows * 4)), the
 *                number of the entries idx[row][0..n_sel) that lie outside
 *                [0, P_t] (each is clamped into the cache and read there, never
 *                out of bounds, so the row's outputs are then wrong); 0 for a
 *                list the selection wrote.  Valid after a call that ran at least
 *                one sparse layer (for the separate-window variant: of the
 *                entries below the window).
 * Returns HS2_OK; HS2_ERR_INVALID_ARG for a null pointer or an unknown region;
 * the status of hs2_workspace_bytes' checks for an invalid shape. */
enum { HS2_WS_LSE2 = 1, HS2_WS_REFINE = 2, HS2_WS_INDEX_CHECK = 3 };
int hs2_workspace_region(const hs2_shape* shape, int32_t n_sparse_layers, int32_t region,
                         size_t* offset, size_t* bytes);

/* ---- Measurement: the device's streaming-read ceiling -----------------------
 * Reads every 16-byte unit of buf (device memory, 16-byte aligned, `bytes`
 * long; only whole 16-byte units are read) once per pass with non-temporal
 * loads, iters passes back to back on `stream`, then synchronises the stream
 * and writes the average milliseconds per pass to *ms_out: bytes / ms is the
 * bandwidth a plain stream reaches, the measured ceiling next to the HBM
 * datasheet peak for the full layer's streaming read.  buf is only read; *sink
 * (device memory, one uint32) is written only if the XOR of everything read
 * equals one fixed constant, which keeps the loads from being optimised away.
 * Not for the serving loop.  Errors: HS2_ERR_INVALID_ARG for null pointers,
 * bytes < 16, iters < 1 or a misaligned buf; HS2_ERR_HIP. */
int hs2_stream_read_ms(const void* buf, size_t bytes, uint32_t* sink, int32_t iters, void* stream,
                       float* ms_out);

/* Human-readable text for a status code (static storage). */
const char* hs2_status_string(int status);

/* hipError_t of the last HS2_ERR_HIP on the calling thread (0 if none). */
int hs2_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H_ */
