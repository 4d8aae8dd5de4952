/*
 * hc.h — C ABI of the sparse-KV hot-cache decode step for one MI355X (gfx950).
 *
 * Source of the method: the page "From 1M Total to 15+ × 1M Contexts: GLM-5.3
 * KV Cache Offloading" (zhuai.tech).  Each decode step the DSA indexer picks
 * the top-2,048 history positions (section "Separate historical capacity from
 * the current working set"); the GPU itself checks its hot slots, hits are read
 * from VRAM, misses are read from registered host RAM, and the gather emits a
 * compact selection for attention (section "Decision three: let the GPU manage
 * the hot cache directly", and its data-flow figure).  Slots used by the
 * current round may not be replaced, and a slot filled in a round is not read
 * by another block of the same gather (section "GPU cache management has
 * hazards too").  Replacement here is a deterministic LRU: the victim is the
 * slot with the oldest last-use step, ties to the lowest slot index.
 *
 * One call of hc_step performs, for every session s and selection group g:
 *   1. exact top-K of the fp32 scores over positions [0, hist_len[s]),
 *      ranked by IEEE-754 totalOrder, ties to the lower position, emitted in
 *      ascending position order;
 *   2. a lookup of each selected position in the group's slot map; hits get
 *      last_use = t;
 *   3. the i-th miss (ascending position) takes the i-th victim in ascending
 *      (last_use, slot) order among slots with last_use != t (LRU; see
 *      HC_REPLACE_* for the other policies); the evicted position leaves the
 *      map;
 *   4. for every layer of the group, the missing rows are copied from pinned
 *      host RAM into the victim slots;
 *   5. every selected row is read from its hot slot and dequantised:
 *      out[j] = bf16_rne((float)int8 latent[j] * (float)fp16 scale[j / 64])
 *      for j < 512, out[512 + k] = RoPE bf16 k for k < 64.
 * t is the number of earlier hc_step calls on the context (0-based).
 *
 * Recent ring (optional, hc_config.ring_rows > 0): new rows made by decode
 * steps enter an HBM ring and reach host RAM through a batched copyback (the
 * page's data-flow figure of "Decision three"; "GPU cache management has
 * hazards too": the ring protects rows that have not reached RAM yet).
 * hc_append adds one position per session; the ring of every (session,
 * layer) holds that session's last ring_rows appended rows.  Once
 * copyback_rows appended rows of a session are not yet in host RAM, one
 * launch copies all of them, for every layer, into the pinned host rows.  A
 * selected position the ring holds — first appended <= p and
 * p >= appended end - ring_rows — is read from the ring and is neither a hit
 * nor a miss: it does not touch the slot map or last-use steps.  hc_flush is
 * the consistency boundary of the page's section "Capacity optimization must
 * survive the session lifecycle": it submits the remaining rows, waits for the
 * copy, and checks the host row count written by the device.
 *
 * Multi-query rounds (hc_config.queries = Q > 1; MTP verification, the
 * page's section "GPU cache management has hazards too"): each of the Q query
 * rows of a round has its own scores and selects its own top-K over the same
 * history.  Steps 2-4 run once on the ascending union of a group's Q
 * selections: a position several queries select is one hit or one miss (one
 * victim, one fill); slots used by any query are pinned; a slot filled in the
 * round is only read in later rounds, and every query row whose position
 * missed — beyond the one that fills the slot — reads host RAM directly.
 * Step 5 gathers each query's rows in its own selection order.  Q = 1 is the
 * single-query step described above.
 *
 * Row format (Q8G64 MLA row, 656 B; the page's payload description): bytes
 * [0,512) int8 latent, [512,528) 8 little-endian fp16 scales (scale g covers
 * latent bytes [64g, 64g+64)), [528,656) 64 little-endian bf16 RoPE values.
 *
 * Layout conventions used below:  S sessions, L layers per session, R layers
 * per selection, G = ceil(L / R) selection groups (layer l is in group l / R),
 * K = top_k, C = cache_slots, Hcap = max_positions.
 *
 * Threading: a context is not thread-safe.  Steps of one context must be issued
 * in order; they may use different streams only if the caller orders them.
 * All entry points return HC_OK or a negative hc_status; none throws.
 */
#ifndef HC_H
#define HC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HC_ROW_BYTES     656   /* bytes of one Q8G64 MLA row                */
#define HC_LATENT_BYTES  512   /* int8 latent bytes, offset 0               */
#define HC_SCALE_OFFSET  512   /* 8 x fp16 group scales                     */
#define HC_ROPE_OFFSET   528   /* 64 x bf16 RoPE                            */
#define HC_OUT_ELEMS     576   /* bf16 values per gathered row (512 + 64)   */
#define HC_MAX_TOPK      4096  /* largest supported top_k                   */
#define HC_MAX_SLOTS     262144 /* largest supported cache_slots            */
#define HC_MAX_SESSIONS  256   /* largest supported n_sessions              */
#define HC_MAX_UNITS     4096  /* largest S * ceil(L / R) (selection units) */
#define HC_MAX_RING_ROWS 65536 /* largest recent ring per (session, layer)  */
#define HC_MAX_QUERIES   16    /* largest number of query rows per round    */
#define HC_MAX_ROUND_ROWS 8192 /* largest queries * top_k                   */
#define HC_NO_APPEND     (~(uint64_t)0)  /* hc_append: this session appends nothing */

/* hc_config.replacement.  LRU: the victim is the slot with the oldest
 * last-use step, ties to the lowest slot.  The two policies of the page's
 * section "GPU cache management has hazards too", as probes: CIRCULAR — a
 * hand moves over the slots and takes the next slot not used in the current
 * step; CLOCK — hits and fills set a slot's reference bit, the hand skips
 * slots used in the current step, clears and skips set bits, and takes the
 * first slot with a clear bit.  Hands start at slot 0 and stop just past
 * their last victim; misses are served in ascending position order. */
#define HC_REPLACE_LRU      0
#define HC_REPLACE_CIRCULAR 1
#define HC_REPLACE_CLOCK    2

/* Per-unit trace record: HC_TRACE_INTS(Q * K) int32 values per (session,
 * group), units ordered u = s * G + g, describing the round's selection
 * union (for Q = 1, the selection itself; N = n_hit + n_miss + n_ring entries
 * in ascending position order, below written with K meaning Q * K).  Layout:
 *   [0] n_hit   [1] n_miss   [2] n_evict (victims whose slot held a position)
 *   [3] n_ring  (selected rows read from the recent ring)
 *   [4] rows the gather read from pinned host RAM over PCIe (656 B each),
 *       counted by the lanes that read them: each missing row of each layer
 *       of the group, and with several query rows each further query row of
 *       a missing position
 *   [5] rows the gather read from HBM (hot slots or the recent ring)
 *   [6] slot fills written (missing rows x layers)
 *   [7] output rows written (Q * K x layers; 0 without an output buffer)
 *   [8 + 0K .. 8 + 1K)  slot of union entry j after the step (ascending
 *                       position); C + p % ring_rows for a row read from the
 *                       ring; -1 past the N entries
 *   [8 + 1K .. 8 + 2K)  miss_pos: missing positions, ascending; -1 past n_miss
 *   [8 + 2K .. 8 + 3K)  victim slot paired with miss i; -1 past n_miss
 *   [8 + 3K .. 8 + 4K)  position evicted from that slot, -1 if it was empty
 * The counts [4]-[7] make the data movement itself observable (page "Making
 * KV offload correct", section "What I tested and what each check could
 * show"); requesting a trace costs a few atomic adds per workgroup. */
#define HC_TRACE_HEADER  8
#define HC_TRACE_INTS(k) (HC_TRACE_HEADER + 4 * (k))

/* Kernel stages timed by hc_profile_read, in launch order. */
#define HC_STAGE_TOPK_SCAN   0  /* score scan: key histogram + candidates   */
#define HC_STAGE_SELECT      1  /* exact cut, lookup, miss compaction, LRU  */
#define HC_STAGE_GATHER      2  /* hits from HBM slots, misses from host RAM
                                   (also written into their victim slots),
                                   dequantised into the bf16 buffer          */
#define HC_NUM_STAGES        3

typedef enum {
  HC_OK      = 0,
  HC_E_INVAL = -1,  /* bad argument or configuration; nothing was changed   */
  HC_E_NOMEM = -2,  /* workspace too small or host allocation failed        */
  HC_E_HIP   = -3,  /* a HIP call failed; the context is now poisoned       */
  HC_E_STATE = -4,  /* the context is poisoned; only hc_destroy is allowed  */
  HC_E_CONSISTENCY = -5, /* hc_flush: a host row count differs from the
                            logical row count                               */
  HC_E_DEVICE = -6       /* a kernel found the context's device state
                            inconsistent (corrupted workspace: counters, slot
                            maps or LRU queue); the context is now poisoned.
                            Reported by the first check after the kernel has
                            completed: hc_step and hc_append at their call,
                            hc_flush and hc_export_state after their wait    */
} hc_status;

typedef struct hc_config {
  uint32_t struct_size;       /* sizeof(hc_config); the sizes without the ring
                                 fields (40) or without `queries` (48) are
                                 accepted: no ring, one query                   */
  uint32_t n_sessions;        /* S, 1 <= S <= HC_MAX_SESSIONS                   */
  uint32_t n_layers;          /* L >= 1 layers per session                      */
  uint32_t layers_per_select; /* R >= 1; S * ceil(L / R) <= HC_MAX_UNITS        */
  uint32_t cache_slots;       /* C, top_k <= C <= HC_MAX_SLOTS                  */
  uint32_t top_k;             /* K, 1 <= K <= HC_MAX_TOPK                       */
  uint64_t max_positions;     /* Hcap: host rows per (session, layer),
                                 K <= Hcap <= 2^31 - 2^19                       */
  int32_t  device;            /* HIP device ordinal                             */
  uint32_t flags;             /* must be 0                                      */
  uint32_t ring_rows;         /* recent ring rows per (session, layer); 0 = no
                                 ring (the caller writes every host row),
                                 else <= HC_MAX_RING_ROWS                       */
  uint32_t copyback_rows;     /* rows per copyback batch, 1 <= copyback_rows <=
                                 ring_rows (0 when ring_rows is 0)              */
  uint32_t queries;           /* Q query rows per round, 0 or 1 = one query;
                                 Q <= HC_MAX_QUERIES, Q * K <= HC_MAX_ROUND_ROWS,
                                 Q * K <= C; the struct without this field
                                 (48 B) means Q = 1                             */
  uint32_t replacement;       /* HC_REPLACE_* (0 = LRU)                         */
} hc_config;

typedef struct hc_ctx hc_ctx;

/* Exact device-workspace size in bytes for cfg (slot maps, LRU order, score
 * scan entries, and the S*L*C hot rows).  HC_E_INVAL for an invalid cfg.
 * Exact sizes rather than pooled over-reservation follow page "From 1M Total
 * to 15+ x 1M Contexts: GLM-5.3 KV Cache Offloading", section "Ten sessions
 * exposed a physical-allocation problem" (memory is sized to what a context
 * actually needs). */
hc_status hc_workspace_bytes(const hc_config* cfg, uint64_t* bytes);

/* Creates a context on cfg->device (page "Making KV offload correct", section
 * "A grouped allocation is a transaction": the context's allocations succeed
 * or fail together).  dev_workspace: caller-owned device memory
 * of at least hc_workspace_bytes bytes, 256-B aligned, that the caller keeps
 * alive and untouched until hc_destroy returns.  The library allocates the
 * pinned host row store itself: S*L buffers of Hcap*656 B (hipHostMalloc,
 * mapped), and initialises the workspace (all caches empty) before returning.
 * All-or-nothing: on failure nothing stays allocated and *out is NULL. */
hc_status hc_create(const hc_config* cfg, void* dev_workspace, uint64_t ws_bytes,
                    hc_ctx** out);

/* Host pointer to the pinned row store of (session, layer): Hcap rows of
 * HC_ROW_BYTES, row p at offset p * 656.  Owned by the library, valid until
 * hc_destroy.  The caller writes row p before the first hc_step whose
 * hist_len exceeds p and never changes it afterwards — except rows at or
 * beyond the session's first hc_append position, which only the library's
 * copyback writes.  NULL on a bad index. */
uint8_t* hc_host_rows(hc_ctx* ctx, uint32_t session, uint32_t layer);

/* One decode step (round), enqueued on `stream` (a hipStream_t; NULL = default
 * stream).  Q = queries (1 if not set).
 *   d_scores     device fp32 [S][G][Q][score_stride]; query (s,g,q) uses
 *                entries [0, hist_len[s]).
 *   score_stride elements between units, >= max_s hist_len[s].
 *   hist_len     host uint64 [S]: positions in each session's history this
 *                step; K <= hist_len[s] <= Hcap, never smaller than at the
 *                previous step, and at most the end of the appended
 *                positions once the session has appended.
 *   d_out        device bf16 bits [S][L][Q][K][576], rows in selection order;
 *                NULL: the step only fetches the missing rows into their slots
 *                (no gathered output), for hc_attend_cached.
 *   d_sel        device int32 [S][G][Q][K]: selected positions, ascending.
 *   d_trace      NULL, or device int32 [S*G][HC_TRACE_INTS(Q*K)] (see above).
 * Asynchronous: results are valid once the stream has completed the step.
 * All arguments are checked before anything is enqueued; a rejected call
 * (HC_E_INVAL) changes nothing.  A HIP launch failure returns HC_E_HIP and
 * poisons the context. */
hc_status hc_step(hc_ctx* ctx, void* stream, const float* d_scores,
                  uint64_t score_stride, const uint64_t* hist_len,
                  uint16_t* d_out, int32_t* d_sel, int32_t* d_trace);

/* Appends one position per session to the recent ring, enqueued on `stream`.
 *   d_rows  device [S][L][656], 16-B aligned: row of position pos[s] for every
 *           layer of session s (sessions skipped by HC_NO_APPEND are ignored).
 *   pos     host uint64 [S]: the session's first call fixes its first appended
 *           position (>= every hist_len it has had, < Hcap); later calls must
 *           continue it (previous pos[s] + 1), or pass HC_NO_APPEND.
 * When a session then has copyback_rows appended rows that are not in host
 * RAM yet, one launch copies all such rows of all sessions and layers to the
 * pinned host rows (GPU stores over PCIe), after which they are in host RAM
 * for every later operation on the stream.  Asynchronous; all arguments are
 * checked before anything is enqueued (HC_E_INVAL changes nothing); HC_E_INVAL
 * also when the context has no ring.  d_rows may be reused once the stream
 * has passed this call. */
hc_status hc_append(hc_ctx* ctx, void* stream, const uint8_t* d_rows, const uint64_t* pos);

/* Consistency boundary: enqueues the copyback of every appended row not yet
 * in host RAM, waits until the stream has completed it (and everything before
 * it), then reads the per-session host row counts the device wrote after the
 * copies (one past the last appended position in host RAM; 0 for a session
 * that has not appended) into host_count[S] if non-NULL.  HC_OK if every
 * appended session's count equals its appended end, else HC_E_CONSISTENCY. */
hc_status hc_flush(hc_ctx* ctx, void* stream, uint64_t* host_count);

/* MLA decode attention over the last step's selection (the consumer of the
 * gather; the page's data-flow figure of "Decision three": the compact
 * selection feeds GPU attention).  For every session, layer, query row q and
 * head h: z_i = scale * <query, row_i> over the 576 values of each selected
 * row (512 latent + 64 RoPE, as the gather writes them), w = softmax(z) over
 * the K rows, out = sum_i w_i * (the row's 512 latent values).  bf16 matrix
 * products on the matrix cores with fp32 accumulation; the softmax weights
 * are rounded to bf16 for the second product.
 *   d_q      device bf16 bits [S][L][Q][heads][576], 16-B aligned.
 *   heads    a multiple of 64, at most 4096.
 *   d_work   caller-owned device scratch of hc_attend_workspace_bytes(heads),
 *            16-B aligned.
 *   d_out    device fp32 [S][L][Q][heads][512], 16-B aligned.
 * hc_attend reads the rows from d_rows, the bf16 [S][L][Q][K][576] output of
 * the last hc_step; hc_attend_cached reads them from the hot slots, the recent
 * ring and host RAM (a further query row of a miss), dequantising on the way,
 * so a step with d_out = NULL plus hc_attend_cached never writes the bf16
 * buffer.  Both give the same result bit for bit.  Asynchronous on `stream`;
 * HC_E_INVAL before any hc_step or for a pointer that is NULL or not aligned
 * as stated; HC_E_NOMEM if work_bytes is too small. */
hc_status hc_attend_workspace_bytes(const hc_ctx* ctx, uint32_t heads, uint64_t* bytes);
hc_status hc_attend(hc_ctx* ctx, void* stream, const uint16_t* d_q, uint32_t heads, float scale,
                    const uint16_t* d_rows, void* d_work, uint64_t work_bytes, float* d_out);
hc_status hc_attend_cached(hc_ctx* ctx, void* stream, const uint16_t* d_q, uint32_t heads,
                           float scale, void* d_work, uint64_t work_bytes, float* d_out);

/* The attention of hc_attend_cached for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same result bit for bit, with
 * the split partials in a scratch array the library holds in device memory
 * (HC_ATTEND_STATIC_BYTES per GPU, for the life of the process) instead of a
 * caller-owned d_work.  No allocation of any kind is made.  HC_E_NOMEM if
 * hc_attend_workspace_bytes(ctx, heads) exceeds HC_ATTEND_STATIC_BYTES (the
 * 78-layer, 64-head, top-2,048 attention needs 30.9 MiB).  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other contexts, other threads) race and give wrong results; calls ordered
 * on one stream do not.  Other arguments and errors as hc_attend_cached. */
#define HC_ATTEND_STATIC_BYTES (32ull << 20)
hc_status hc_attend_cached_noalloc(hc_ctx* ctx, void* stream, const uint16_t* d_q,
                                   uint32_t heads, float scale, float* d_out);

/* Synchronous snapshot for tests: waits for all enqueued steps, then copies
 * the state that layer `layer` of `session` sees into host buffers:
 * slot2pos[C] and last_use[C] (-1 = empty / never used), pos2slot[Hcap] if
 * non-NULL, and the layer's hot rows [C][656] if hot_rows is non-NULL (the
 * bytes of an empty slot are whatever the workspace held: unspecified). */
hc_status hc_export_state(hc_ctx* ctx, uint32_t session, uint32_t layer,
                          int32_t* slot2pos, int32_t* last_use,
                          int32_t* pos2slot, uint8_t* hot_rows);

/* Per-stage kernel timing: a pair of HIP events per stage, attached to the
 * stage's first and last kernel dispatch on the step's stream, so that they
 * record the kernels' own begin and end (no event is enqueued between
 * kernels).  hc_profile_enable(ctx, n) arms timing for the next n steps
 * (n = 0 disarms; any earlier timing is dropped).  hc_profile_read waits for
 * the timed steps and returns the summed milliseconds per stage
 * (stage_ms[HC_NUM_STAGES]), the number of timed steps, and, if per_step is
 * non-NULL, the milliseconds of each stage of each step, row-major
 * [step][HC_NUM_STAGES], for at most per_step_cap steps. */
hc_status hc_profile_enable(hc_ctx* ctx, uint32_t max_steps);
hc_status hc_profile_read(hc_ctx* ctx, double* stage_ms, double* per_step,
                          uint64_t per_step_cap, uint64_t* n_steps);

/* Number of steps issued so far (the t the next hc_step will use). */
hc_status hc_steps_done(const hc_ctx* ctx, uint64_t* n);

/* Waits for every step the context enqueued, then frees the pinned host store
 * and the context (page "Making KV offload correct", section "Response
 * completion is not copy completion": memory a queued copy still uses is not
 * released before that copy has finished).  The caller's workspace is not
 * freed.  NULL-safe. */
hc_status hc_destroy(hc_ctx* ctx);

const char* hc_status_str(hc_status s);

#ifdef __cplusplus
}
#endif
#endif /* HC_H */
