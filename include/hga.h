/*
 * hga.h -- C ABI of the MI355X (gfx950) Hierarchical Global Attention hot path.
 *
 * HGA replaces dense causal attention of a pretrained GQA model without new
 * weights: the projected Q/K/V go in, the attention output comes out (HGA
 * technical summary, gist.science, sections "Methodologie" and
 * "Belangrijkste Bijdragen", item 1).  Inside, each query routes in two
 * levels over RoPE-aware key summaries, and then attends exactly over the
 * token K/V of the selected set ("Kernmechanisme", items 1-4).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, C-contiguous, in the layouts written next
 *     to each argument.  Pointers are device pointers unless stated.
 *   - The caller owns all memory.  No entry point allocates or frees memory;
 *     scratch space comes from the caller's workspace `ws` (see
 *     hga_workspace_bytes).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously.  No entry point synchronises.
 *   - Arguments are checked on the host before anything is launched.  On any
 *     error the call returns a status other than HGA_OK and launches nothing.
 *     A HIP launch failure returns HGA_ERR_HIP.
 *   - Query positions live in device memory (q_pos0), so that a captured
 *     graph can be replayed for successive positions.  The kernels check
 *     them; a unit whose position is invalid gets n_sel = -1 from hga_route
 *     and NaN outputs from hga_attend.
 *   - Supported shapes: head_dim 64 or 128; chunk_size 64 with 4 groups of
 *     16 tokens; n_q_heads / n_kv_heads in {1, 2, 4, 8}.  Other shapes
 *     return HGA_ERR_UNSUPPORTED (there is no slow fallback path).
 *   - A workspace serves one stream at a time.  Two calls that may run
 *     concurrently need two workspaces.
 *   - No global mutable state (save the per-device address of the static
 *     scratch of hga_decode_step_noalloc, set once under a lock); the library
 *     is safe to call from several host threads on different streams.
 */
#ifndef HGA_H_
#define HGA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HGA_OK = 0,
  HGA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad enum */
  HGA_ERR_UNSUPPORTED = 2,      /* valid config outside the supported shapes */
  HGA_ERR_WORKSPACE_TOO_SMALL = 3,
  HGA_ERR_OUT_OF_RANGE = 4,     /* positions beyond a capacity, max_sel too small */
  HGA_ERR_HIP = 5               /* a HIP runtime call or launch failed */
} hga_status;

typedef enum { HGA_F32 = 0, HGA_BF16 = 1 } hga_dtype;

/* Where hga_attend reads K/V for a selected group. */
typedef enum {
  HGA_SRC_POOL = 0,        /* group id gid occupies rows gid*16 .. of a [cap][d] pool */
  HGA_SRC_WORKING_SET = 1  /* list slot s occupies rows s*16 .. of a [max_sel*16][d] set */
} hga_src_layout;

/* Which part of the selected list a call covers (the pinned-host tier
 * attends the resident window groups and the transferred routed groups in two
 * calls, then merges them with hga_merge_partials). */
typedef enum {
  HGA_PART_ALL = 0,
  HGA_PART_WINDOWS = 1,    /* sink, local and current-chunk groups */
  HGA_PART_ROUTED = 2      /* groups chosen by the two-level routing */
} hga_part;

/* Phases of hga_prefill_prompt (bit mask). */
typedef enum {
  HGA_PROMPT_APPEND = 1,   /* pool rows and chunk/group summaries of the prompt */
  HGA_PROMPT_ROUTE = 2,    /* selected list of every query chunk */
  HGA_PROMPT_ATTEND = 4,   /* attention of every query chunk over its list */
  HGA_PROMPT_ALL = 7
} hga_prompt_phase;

typedef struct {
  int32_t head_dim;        /* d */
  int32_t n_q_heads;       /* Hq */
  int32_t n_kv_heads;      /* Hkv; query head h reads KV head h / (Hq/Hkv) */
  int32_t chunk_size;      /* C: tokens per chunk */
  int32_t groups_per_chunk;/* G: contiguous groups of C/G tokens */
  int32_t n_sink_chunks;   /* leading chunks that are always visible */
  int32_t n_local_chunks;  /* chunks just before the current one, always visible */
  int32_t topk_chunks;     /* level-1 budget k_c */
  int32_t topk_groups;     /* level-2 budget k_g (global over the k_c*G groups) */
  double rope_theta;       /* RoPE base: omega_j = theta^(-2j/d) for pair j */
  double hf_wavelength;    /* pair j is high-frequency iff 2*pi/omega_j < this */
  int32_t qkv_dtype;       /* hga_dtype of q, k, v and of the K/V pool */
  int32_t rep_position;    /* position the low-frequency pairs of a span's summary are
                              rotated to: 0 = the midpoint a + (n-1)/2, 1 = a + n/2 */
  int32_t route_per_head;  /* 0: one selected list per (sequence, KV head), routed with
                              the mean of its query heads; 1: one list per (sequence,
                              query head), routed with that head's query alone.  With 1
                              the list arrays are [B][Hq][...] instead of [B][Hkv][...],
                              a working set [B][Hq][max_sel*16][d]; hga_prefill_prompt
                              and hga_attend_tiered return HGA_ERR_UNSUPPORTED */
  int32_t rope_style;      /* RoPE pairs: 0 = (x_j, x_{j+d/2}) (half-split), 1 =
                              (x_{2j}, x_{2j+1}) (interleaved); the pool keys, the
                              summaries and the rotated queries follow it */
  int32_t pool_dtype;      /* 0: the K/V pool holds qkv_dtype; 1: the FP8 pool (bf16
                              inputs, head_dim 128): each (token, KV head) row of the
                              rotated keys and of the values as OCP E4M3FN codes times
                              the smallest power of two s with max|x| <= 448 s.  A pool
                              buffer then holds the codes, [B][Hkv][cap][d] bytes (V in
                              transposed group blocks), followed by the row scales,
                              [B][Hkv][cap] fp32.  Every entry point takes it; a
                              working set (hga_gather, hga_warm_gather) then holds
                              the codes [B][lists][max_sel*16][d] bytes followed by
                              the row scales [B][lists][max_sel*16] fp32, and a
                              warm cache the codes [B][lists][n_warm*16][d] bytes
                              followed by [B][lists][n_warm*16] fp32 scales */
  int32_t route_pool;      /* routing query of a list's query heads ("Kernmechanisme"
                              items 2-3 leave the pooling open): 0 = their mean
                              (over heads and query tokens); 1 = max pooling: each
                              head's query is the mean over the query tokens, and a
                              candidate chunk or group scores the largest of the
                              heads' scores.  Equal to 0 with one head per list */
} hga_config;

/* Checks a configuration (host only).  HGA_OK, HGA_ERR_INVALID_ARGUMENT for
 * inconsistent values (d odd, Hq % Hkv != 0, C % G != 0, negative budgets,
 * theta <= 1, rep_position, route_per_head, rope_style, pool_dtype or
 * route_pool outside {0, 1}),
 * HGA_ERR_UNSUPPORTED for valid shapes this build does not implement. */
hga_status hga_validate(const hga_config* cfg);

/* Worst-case length of a selected-group list for queries of up to max_lq
 * tokens: (n_sink + n_local + 1) * G + topk_groups. */
hga_status hga_max_selected(const hga_config* cfg, int32_t max_lq, int32_t* max_sel);

/* Bytes of device workspace needed by hga_route, hga_attend and
 * hga_attend_tiered for batch B,
 * contexts up to max_ctx tokens and up to max_lq query tokens per call.  The
 * workspace carries nothing from one call to the next (route keeps its
 * scores there between its two kernels, attend its per-split partials), so
 * it needs no initialisation; one workspace may serve route and attend on
 * the same stream. */
hga_status hga_workspace_bytes(const hga_config* cfg, int32_t B, int32_t max_ctx, int32_t max_lq,
                               size_t* bytes);

/* Zero-fills a buffer (e.g. a workspace) with a kernel; no hipMemset node, so
 * it may be captured in a graph. */
hga_status hga_workspace_reset(void* ws, size_t ws_bytes, void* stream);

/* Pool append and RoPE-aware summaries ("Kernmechanisme" items 3 and 4).
 *   k_raw  [B][Hkv][n_tok][d] raw (pre-RoPE) projected keys of positions
 *          pos0 .. pos0+n_tok-1, qkv_dtype
 *   v_new  [B][Hkv][n_tok][d] values of those positions (may be NULL when
 *          k_pool is NULL)
 *   k_pool  [B][Hkv][pool_cap][d] qkv_dtype: row p receives RoPE(k_raw, p)
 *          rounded once to qkv_dtype (round-to-nearest-even).
 *   v_pool  [B][Hkv][pool_cap/16][d][16] qkv_dtype: each 16-token group is
 *          stored transposed, so token p, dim e sits at
 *          [(p/16)*d + e]*16 + p%16 of its unit; values unchanged.
 *          Both pools: device memory or pinned host memory (written over
 *          PCIe); pool_cap a multiple of 16.  NULL (both) skips the append.
 *   chunk_sum [B][Hkv][max_chunks][d] fp32, group_sum [B][Hkv][max_chunks*G][d]
 *          fp32.  For every chunk that lies entirely inside the range, its
 *          chunk summary and its G group summaries are written: for pair j,
 *          high-frequency pairs take the mean of the per-token rotated pair,
 *          low-frequency pairs take the mean raw pair rotated to the span's
 *          representative position (cfg->rep_position: the midpoint
 *          a + (n-1)/2, or a + n/2).  NULL (both) skips the summaries.
 * A decode step that completes a chunk passes that chunk's 64 raw keys (the
 * rows already in the pool are rewritten with identical values).
 * Errors: HGA_ERR_OUT_OF_RANGE if pos0 + n_tok > pool_cap or a completed
 * chunk index >= max_chunks. */
hga_status hga_build_summaries(const hga_config* cfg, int32_t B, const void* k_raw,
                               const void* v_new, int32_t pos0, int32_t n_tok, void* k_pool,
                               void* v_pool, int32_t pool_cap, float* chunk_sum,
                               float* group_sum, int32_t max_chunks, void* stream);

/* Two-level routing ("Kernmechanisme" item 2) for each (sequence b, KV head),
 * or, with cfg->route_per_head, each (sequence b, query head): the list arrays
 * below are then [B][Hq][...].
 *   q_raw   [B][Hq][lq][d] raw queries of positions q_pos0[b] .. +lq-1, which
 *           must lie in one chunk c_t (device q_pos0 [B] int32)
 *   The routing query is the mean over the KV head's query heads (or the one
 *   query head) and the query tokens of RoPE(q, position).  Level 1 scores the candidate chunks
 *   n_sink <= c < c_t - n_local as qbar . chunk_sum[c] / sqrt(d) and keeps
 *   the top_k_c by (score desc, id asc); level 2 scores the G groups of each
 *   kept chunk the same way and keeps the global top k_g.  Summaries of all
 *   candidate chunks must have been built.
 *   sel_groups [B][Hkv][max_sel] int32 receives, in ascending order, the
 *           sink groups, the routed groups, the local groups and the current
 *           chunk's groups up to the last query token; n_sel [B][Hkv] their
 *           count (-1 for an invalid position: negative, tokens spanning two
 *           chunks, or a query chunk at or beyond max_chunks).
 *   chunk_scores_opt [B][Hkv][max_chunks] fp64 (nullable): level-1 score of
 *           every candidate chunk, at its chunk index.
 * Errors: HGA_ERR_OUT_OF_RANGE if max_sel < hga_max_selected(). */
hga_status hga_route(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                     const int32_t* q_pos0, const float* chunk_sum, const float* group_sum,
                     int32_t max_chunks, int32_t* sel_groups, int32_t* n_sel, int32_t max_sel,
                     double* chunk_scores_opt, void* ws, size_t ws_bytes, void* stream);

/* Gather of the selected token K/V into a compact working set: after routing,
 * the original token-level keys and values of the selected groups are fetched
 * into accelerator memory for the exact attention (HGA technical summary,
 * gist.science, "Kernmechanisme" item 4), from the device pool or, for the
 * cold tier of "Geheugenarchitectuur" (full K/V history in host RAM), from a
 * pinned host pool over PCIe.
 *   k_pool, v_pool as written by hga_build_summaries (pool_cap a multiple of
 *           16): device memory, or pinned host memory (pool_is_host = 1, read
 *           directly over PCIe).
 *   k_ws, v_ws [B][lists][max_sel*16][d] elements (lists = Hkv, or Hq with
 *           route_per_head = 1; caller-owned, and the library cannot check
 *           its size): list slot s of list (b, h) receives the 16*d block of
 *           group sel_groups[b][h][s] (K rows; V in the pool's transposed
 *           group layout).  Bit-exact copy.
 *   part    HGA_PART_ALL copies every slot; HGA_PART_ROUTED only the routed
 *           slots; HGA_PART_WINDOWS only the window slots (q_pos0 tells them
 *           apart; it may be NULL for HGA_PART_ALL).
 * Errors: HGA_ERR_INVALID_ARGUMENT if pool_is_host is set and the pool is
 * not pinned host memory. */
hga_status hga_gather(const hga_config* cfg, int32_t B, const void* k_pool, const void* v_pool,
                      int32_t pool_cap, int32_t pool_is_host, const int32_t* sel_groups,
                      const int32_t* n_sel, int32_t max_sel, const int32_t* q_pos0, int32_t part,
                      void* k_ws, void* v_ws, void* stream);

/* Exact attention over the selected set ("Kernmechanisme" item 4): for query
 * head h (KV head h / (Hq/Hkv)) and query token tau,
 *   out = sum_p softmax_p(RoPE(q, tau) . K[p] / sqrt(d)) V[p]
 * over the tokens p <= tau of the selected groups (restricted to `part`).
 *   k_src, v_src  the pool written by hga_build_summaries (HGA_SRC_POOL,
 *           src_cap tokens per unit, a multiple of 16) or a working set from
 *           hga_gather (HGA_SRC_WORKING_SET, max_sel*16 tokens)
 *   out     [B][Hq][lq][d] fp32
 *   lse_opt [B][Hq][lq] fp32 natural-log sum of exp of the logits (nullable);
 *           with hga_merge_partials it joins results over disjoint parts.
 * Both shapes contract on the matrix cores: decode (lq < 16) takes the Hg
 * query heads of a KV head as the columns of one MFMA block; 16 <= lq <= 64
 * (the query tokens of one chunk; the page's "Experimentele Resultaten"
 * report a fused prefill speed-up) runs the chunked-prefill kernel, which
 * needs head_dim 128 and bf16 (else HGA_ERR_UNSUPPORTED).  Query tokens must lie in one chunk:
 * (q_pos0 % chunk_size) + lq <= chunk_size, checked on the device (NaN
 * outputs otherwise).  Pool rows after the last query token are never read
 * into the result, whatever they hold.
 * Errors: HGA_ERR_UNSUPPORTED for max_sel > 256. */
hga_status hga_attend(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                      const int32_t* q_pos0, const void* k_src, const void* v_src,
                      int32_t src_layout, int32_t src_cap, const int32_t* sel_groups,
                      const int32_t* n_sel, int32_t max_sel, int32_t part, float* out,
                      float* lse_opt, void* ws, size_t ws_bytes, void* stream);

/* One fused decode step: for each sequence b, the query token at position
 * q_pos0[b] (device) is appended, routed and attended, in four launches
 * instead of the six of the separate calls:
 *   1. level-1 scores of every candidate chunk (as hga_route);
 *   2. level-1 / level-2 selection and the list (as hga_route), and, in extra
 *      workgroups of the same launch, the token work: its rotated key and its
 *      value into the pool (bit-identical to hga_build_summaries with
 *      n_tok = 1), its raw key into the chunk staging rows, and, when the
 *      token is the last of its chunk, that chunk's summaries (as
 *      hga_build_summaries over the chunk).  The current chunk is never a
 *      routing candidate, so this work and the routing do not interact;
 *   3. attention over the list, 4. the split merge (as hga_attend).
 *   q_raw       [B][Hq][1][d] raw query
 *   k_new, v_new [B][Hkv][d] raw key and value of the token at q_pos0[b]
 *   k_stage     [B][Hkv][chunk_size][d] qkv_dtype, caller-owned and kept
 *               across steps: row p % chunk_size holds the raw key of position
 *               p of the current chunk.  Before the first step of a chunk the
 *               caller (or the previous steps) must have written the rows of
 *               the chunk's earlier positions.
 *   other arguments as hga_build_summaries, hga_route and hga_attend; the
 *   workspace is shared by the route and attend phases.
 * An unusable position (negative, outside the pool or beyond max_chunks
 * chunks) gives n_sel = -1 and NaN outputs and writes nothing.  Errors: as
 * hga_route and hga_attend.  hga_decode_step is hga_prefill_step with lq = 1. */
hga_status hga_decode_step(const hga_config* cfg, int32_t B, const void* q_raw, const void* k_new,
                           const void* v_new, const int32_t* q_pos0, void* k_pool, void* v_pool,
                           int32_t pool_cap, void* k_stage, float* chunk_sum, float* group_sum,
                           int32_t max_chunks, int32_t* sel_groups, int32_t* n_sel,
                           int32_t max_sel, float* out, float* lse_opt, void* ws, size_t ws_bytes,
                           void* stream);

/* Bytes of the static device scratch array behind hga_decode_step_noalloc. */
#define HGA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* hga_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, results and errors, except that there is no workspace
 * argument.  Its scratch (the routing scores and the attention partials)
 * lives in a static device array of HGA_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on every GPU it runs on until the process ends; the array of
 * the current device (hipGetDevice) is used, so `stream` must belong to that
 * device.  The call allocates and frees nothing.  Every call on one GPU shares
 * that GPU's array and nothing in it carries from one call to the next, so
 * calls that may overlap on one GPU (concurrent streams, several host
 * threads) race: serialise them.
 * Errors: as hga_decode_step; HGA_ERR_WORKSPACE_TOO_SMALL when the scratch
 * the call needs (what hga_workspace_bytes(cfg, B, max_chunks * C, 1) gives)
 * exceeds HGA_NOALLOC_SCRATCH_BYTES (for the 32/4-head, head_dim 128 layer at
 * 64K context that is batch 64 and beyond); HGA_ERR_HIP if the scratch address
 * cannot be obtained. */
hga_status hga_decode_step_noalloc(const hga_config* cfg, int32_t B, const void* q_raw,
                                   const void* k_new, const void* v_new, const int32_t* q_pos0,
                                   void* k_pool, void* v_pool, int32_t pool_cap, void* k_stage,
                                   float* chunk_sum, float* group_sum, int32_t max_chunks,
                                   int32_t* sel_groups, int32_t* n_sel, int32_t max_sel,
                                   float* out, float* lse_opt, void* stream);

/* One fused chunked-prefill step: for each sequence b, the lq query tokens at
 * positions q_pos0[b] .. q_pos0[b] + lq - 1, all inside one chunk, are
 * appended, routed with their pooled query and attended, in the four
 * launches of hga_decode_step.  This is the per-chunk step of the page's
 * chunked prefill (HGA technical summary, "Kernmechanisme" items 2-4: the
 * current chunk's queries route over the chunk summaries and attend the
 * exact K/V of the selected set; "Experimentele Resultaten" reports the
 * speed-up of fusing it).
 *   q_raw        [B][Hq][lq][d] raw queries
 *   k_new, v_new [B][Hkv][lq][d] raw keys and values of the lq tokens
 *   k_stage      as hga_decode_step: rows of the chunk's positions before
 *                q_pos0[b] must hold their raw keys; the call writes the rows
 *                of its own tokens.  When the last token ends its chunk the
 *                chunk's summaries are built (from those rows and the new
 *                keys; in one pass when the step holds the whole chunk).
 *   other arguments as hga_decode_step; ws sized by hga_workspace_bytes with
 *   max_lq >= lq.
 * Results are bit-identical to hga_build_summaries (append of the lq tokens,
 * then the chunk's summaries if it ends), hga_route and hga_attend with the
 * same arguments.  lq >= 16 runs the matrix-core prefill attention, which
 * needs head_dim 128 and bf16 (else HGA_ERR_UNSUPPORTED).
 * Errors: HGA_ERR_INVALID_ARGUMENT for lq outside 1..chunk_size; otherwise as
 * hga_decode_step.  Tokens that would cross a chunk end make the position
 * unusable (n_sel = -1, NaN outputs, nothing written). */
hga_status hga_prefill_step(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                            const void* k_new, const void* v_new, const int32_t* q_pos0,
                            void* k_pool, void* v_pool, int32_t pool_cap, void* k_stage,
                            float* chunk_sum, float* group_sum, int32_t max_chunks,
                            int32_t* sel_groups, int32_t* n_sel, int32_t max_sel, float* out,
                            float* lse_opt, void* ws, size_t ws_bytes, void* stream);

/* Workspace of hga_prefill_prompt for B prompts of T tokens with summary
 * tables of max_chunks rows (host only). */
hga_status hga_prompt_workspace_bytes(const hga_config* cfg, int32_t B, int32_t T,
                                      int32_t max_chunks, size_t* bytes);

/* Whole-prompt chunked prefill: the prompt's T tokens (T a multiple of
 * chunk_size) are appended to the pool with their chunk and group summaries,
 * then every query chunk qc (positions qc*C .. qc*C + C - 1) is routed with
 * its pooled query over the complete chunks before it and attended over its
 * selected list, causally inside its own chunk.  This is the chunked prefill
 * of the page (HGA technical summary, "Kernmechanisme" items 2-4), whose
 * "Experimentele Resultaten" report the speed-up of fusing it: since a query
 * chunk reads only earlier chunks and its own, all query chunks of a prompt
 * are routed by one launch pair and attended by one launch.
 *   q_raw        [B][Hq][T][d] raw queries (bf16)
 *   k_raw, v_raw [B][Hkv][T][d] raw keys and values
 *   k_pool, v_pool, chunk_sum, group_sum: as hga_build_summaries, written by
 *                the append phase (pool_cap >= T, max_chunks >= T / C)
 *   sel_groups   [B][T/C][Hkv][max_sel] list of each query chunk (ascending
 *                group ids), n_sel [B][T/C][Hkv] its length: written by the
 *                route phase, as hga_route for that chunk alone
 *   out          [B][Hq][T][d] fp32, lse_opt [B][Hq][T] (nullable): written by
 *                the attend phase, as hga_attend for that chunk alone up to
 *                fp32 rounding (the softmax runs online over tiles of 8
 *                groups instead of split partials)
 *   phases       HGA_PROMPT_* mask; a phase reads what the earlier phases (of
 *                this call or a previous one) wrote
 *   ws           hga_prompt_workspace_bytes; shared by the phases of one call
 * Needs head_dim 128 and bf16 (the matrix-core attention): else
 * HGA_ERR_UNSUPPORTED.  Errors: HGA_ERR_INVALID_ARGUMENT for T not a
 * multiple of chunk_size, a missing buffer or a bad phase mask;
 * HGA_ERR_OUT_OF_RANGE for T beyond pool_cap or max_chunks, or max_sel below
 * hga_max_selected; HGA_ERR_UNSUPPORTED for max_sel > 256;
 * HGA_ERR_WORKSPACE_TOO_SMALL. */
hga_status hga_prefill_prompt(const hga_config* cfg, int32_t B, int32_t T, const void* q_raw,
                              const void* k_raw, const void* v_raw, void* k_pool, void* v_pool,
                              int32_t pool_cap, float* chunk_sum, float* group_sum,
                              int32_t max_chunks, int32_t* sel_groups, int32_t* n_sel,
                              int32_t max_sel, float* out, float* lse_opt, int32_t phases,
                              void* ws, size_t ws_bytes, void* stream);

/* Host-tier attention (page section "Geheugenarchitectuur": summaries and the
 * always-visible windows are hot in device memory, the full token K/V history
 * is cold in host RAM).  For the list written by hga_route:
 *   stream_b: the routed groups are copied from the pinned host pool over PCIe
 *             into the working set (hga_gather, HGA_PART_ROUTED) and attended
 *             there (hga_attend, HGA_PART_ROUTED, HGA_SRC_WORKING_SET);
 *   stream_a: meanwhile the window groups are attended from the device pool
 *             (HGA_PART_WINDOWS, HGA_SRC_POOL); then stream_a waits for
 *             stream_b and merges the two parts exactly (log-sum-exp).
 * The result equals hga_attend over the whole list (up to fp32 rounding of
 * the merge).  Stream b starts after the work already queued on stream a;
 * when the call returns, out / lse_opt are complete in stream a's order.
 *   k_hot, v_hot   [B][Hkv][hot_cap][d] device pool; only the rows of the
 *                  window groups (sink, local, current chunk up to the last
 *                  query token) are read
 *   k_cold, v_cold [B][Hkv][cold_cap][d] pinned host memory (the full pool)
 *   k_ws, v_ws     [B][Hkv][max_sel*16][d] device working set (routed slots
 *                  are overwritten)
 *   out, lse_opt   as hga_attend
 *   ws             hga_workspace_bytes() of workspace (this call needs room
 *                  for two attention partial sets and two part results)
 * The two-stream form records the caller's two HIP events: ev_fork on
 * stream_a (stream_b waits for it) and ev_join on stream_b (stream_a waits for
 * it before the merge); both are hipEvent_t created by the caller (timing may
 * be disabled), distinct, and not recorded elsewhere while the call's work is
 * queued.  The call creates and destroys nothing.
 * stream_b = NULL selects the one-stream form: for 1..15 query tokens the
 * window part's attention and the PCIe copy of the routed groups run as
 * workgroups of one launch on stream_a (the copy workgroups mostly wait on
 * PCIe, the attention workgroups use the CUs meanwhile), then the routed
 * part and the merge follow on stream_a; no events.  (For 16..64 query
 * tokens the one-stream form runs the parts one after another.)  Both forms
 * give the same bits.
 * Errors: as hga_attend; HGA_ERR_INVALID_ARGUMENT if the cold pool is not
 * pinned host memory, or if stream_b is set and the two events are missing or
 * the same. */
hga_status hga_attend_tiered(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                             const int32_t* q_pos0, const void* k_hot, const void* v_hot,
                             int32_t hot_cap, const void* k_cold, const void* v_cold,
                             int32_t cold_cap, const int32_t* sel_groups, const int32_t* n_sel,
                             int32_t max_sel, void* k_ws, void* v_ws, float* out, float* lse_opt,
                             void* ws, size_t ws_bytes, void* stream_a, void* stream_b,
                             void* ev_fork, void* ev_join);

/* Workspace of hga_warm_gather (host only). */
hga_status hga_warm_workspace_bytes(const hga_config* cfg, int32_t B, int32_t max_sel,
                                    size_t* bytes);

/* Warm tier of a pinned host pool (page section "Geheugenarchitectuur": a
 * bounded LRU cache in device memory holds recently routed data between the
 * hot windows and summaries and the cold host pool).  The cache holds 16-token
 * groups, the unit that routing selects and attention reads: n_warm slots per
 * (sequence, list).  For the routed part of each list written by hga_route
 * (as hga_gather with HGA_PART_ROUTED selects it):
 *   - a group found in the unit's cache is a hit: its stamp becomes `step`;
 *   - the i-th miss in list order takes the i-th least recently used slot
 *     that is not a hit this step (stamp order, ties by slot index, empty
 *     slots first), is copied from the pinned host pool over PCIe into that
 *     slot, and the slot's tag and stamp are rewritten;
 *   - every routed list slot s of the working set receives its group (from
 *     PCIe for a miss, from the cache for a hit), rows 16*s .. of
 *     k_ws / v_ws [B][lists][max_sel*16][d] -- what hga_gather with
 *     HGA_PART_ROUTED would write; window slots are not touched.
 *   k_cold, v_cold  the pool in pinned host memory, as hga_gather
 *   k_warm, v_warm  [B][lists][n_warm][16][d] qkv_dtype (FP8 pool: codes, then
 *                   row scales, as cfg->pool_dtype describes) device memory: slot w
 *                   holds a group's K rows and its V^T block (the pool's
 *                   group layout)
 *   warm_tags [B][lists][n_warm] int32, warm_used [B][lists][n_warm] int32:
 *                   caller-owned state kept across calls; before the first
 *                   call fill warm_tags with -1 and warm_used with 0
 *   n_warm          topk_groups <= n_warm <= 1024 (else HGA_ERR_OUT_OF_RANGE)
 *   step            > 0, larger on every call (the LRU stamp)
 *   hits_opt [B][lists] int32 (nullable): routed groups found in the cache
 *   ws              hga_warm_workspace_bytes() of workspace (the fill plan)
 * Two launches on `stream`; the working set is then ready for hga_attend with
 * HGA_PART_ROUTED and HGA_SRC_WORKING_SET.
 * Errors: HGA_ERR_INVALID_ARGUMENT if the host pool is not pinned or step <= 0;
 * HGA_ERR_UNSUPPORTED for max_sel > 256. */
hga_status hga_warm_gather(const hga_config* cfg, int32_t B, const void* k_cold, const void* v_cold,
                           int32_t cold_cap, const int32_t* sel_groups, const int32_t* n_sel,
                           int32_t max_sel, const int32_t* q_pos0, void* k_warm, void* v_warm,
                           int32_t* warm_tags, int32_t* warm_used, int32_t n_warm, int32_t step,
                           void* k_ws, void* v_ws, int32_t* hits_opt, void* ws, size_t ws_bytes,
                           void* stream);

/* Exact merge of two attention results over disjoint token sets, so that
 * attention computed in parts equals softmax attention over their union (the
 * exactness of "Kernmechanisme" item 4 when the hot windows and the cold
 * routed groups of "Geheugenarchitectuur" are attended separately; HGA
 * technical summary, gist.science):
 * out = (e^{lse_a} out_a + e^{lse_b} out_b) / (e^{lse_a} + e^{lse_b}),
 * lse_out = log(e^{lse_a} + e^{lse_b}) (lse_out nullable).  Rows are
 * [B][Hq][lq], each of d fp32 values.  out may alias out_a or out_b. */
hga_status hga_merge_partials(const hga_config* cfg, int32_t B, int32_t lq, const float* out_a,
                              const float* lse_a, const float* out_b, const float* lse_b,
                              float* out, float* lse_out, void* stream);

const char* hga_status_string(hga_status s);
int32_t hga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H_ */
