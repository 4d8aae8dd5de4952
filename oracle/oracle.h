/*
 * oracle.h — plain CPU oracle of the sparse-KV hot-cache decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * It follows the page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache
 * Offloading" (zhuai.tech): sections "Separate historical capacity from the
 * current working set" (top-2,048 selection, 656-B Q8G64 rows), "Decision
 * three: let the GPU manage the hot cache directly" (hit/miss gather into a
 * compact selection) and "GPU cache management has hazards too" (slots used in
 * the current round are not replaced).  Replacement is LRU by last-use step
 * with ties to the lowest slot.  Every function is the plain definition: a
 * full sort for top-K, a linear scan per miss for the LRU victim, and exact
 * double arithmetic rounded to bf16 for the dequantisation.
 *
 * Parity pins live in tests/test_oracle_*.py; every function here is pinned.
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stdint.h>

#define ORC_ROW_BYTES 656
#define ORC_OUT_ELEMS 576

/* Exact top-K of scores[0..H): rank by IEEE-754 totalOrder descending, ties to
 * the lower position, then emit the K positions in ascending order.
 * Returns 0, or -1 if K < 1 or K > H. */
int orc_topk(const float* scores, int64_t H, int32_t K, int32_t* sel);

/* One dequantised element: bf16 bits of round-to-nearest-even of the exact
 * product q * value(scale), value(scale) being the fp16 number with those bits. */
uint16_t orc_dequant_elem(int8_t q, uint16_t scale_bits);

/* One 656-B row to 576 bf16 values (512 dequantised latent + 64 RoPE copied). */
void orc_dequant_row(const uint8_t* row, uint16_t* out);

/* Fills table[q + 128][scale_bits] for all 256 int8 q and all 65,536 scale bit
 * patterns (non-finite scales included; every NaN result is the canonical
 * 0x7FC0, whatever the signs of q and the scale). */
void orc_dequant_table(uint16_t* table);

/* Recent ring of one (session, layer): rows appended by decode steps live
 * here until a batched copyback writes them to host RAM.  It holds the last
 * `rows` appended rows; after an append, once `batch` appended rows are not
 * yet in host RAM, all of them are copied (batch <= rows, so a ring entry is
 * in host RAM before it is reused). */
typedef struct orc_ring orc_ring;

orc_ring* orc_ring_new(int32_t rows, int32_t batch);
void      orc_ring_free(orc_ring* r);

/* Appends the row of position p: the first append fixes the ring's first
 * position, later ones must continue it (p = previous p + 1).  host_rows is
 * the (session, layer)'s host row store, written by copybacks.  Returns 0, or
 * -1 for an out-of-order position. */
int orc_ring_append(orc_ring* r, int64_t p, const uint8_t* row, uint8_t* host_rows);

/* Copies every appended row not yet in host RAM; returns the host row
 * frontier (one past the last appended row in host RAM; 0 if none). */
int64_t orc_ring_flush(orc_ring* r, uint8_t* host_rows);

/* The ring's row of position p, or NULL if the ring does not hold p (r may
 * be NULL: no ring). */
const uint8_t* orc_ring_row(const orc_ring* r, int64_t p);

/* Host row frontier without copying (0 before the first append). */
int64_t orc_ring_copied(const orc_ring* r);

/* MLA decode attention over K gathered rows (the consumer of the gather):
 * q [H][576] and rows [K][576] are bf16 bit patterns (rows as the gather
 * writes them: 512 dequantised latent values, 64 RoPE values).  For each head
 * h: z_i = scale * <q[h], row_i> over all 576 values, w = softmax(z),
 * out[h][d] = sum_i w_i * row_i[d] for the 512 latent values (double). */
void orc_attend(const uint16_t* q, const uint16_t* rows, int32_t H, int32_t K, double scale,
                double* out);

/* LRU hot cache of one (session, layer). */
typedef struct orc_cache orc_cache;

typedef struct orc_step_info {
  int32_t n_hit, n_miss, n_evict;
  int32_t* slot;       /* [K]: slot of sel[i] after the step; C + (p % ring
                          rows) for a row read from the recent ring         */
  int32_t* miss_pos;   /* [K]: misses in processing order (ascending pos)    */
  int32_t* victim;     /* [K]: slot given to miss i                          */
  int32_t* evicted;    /* [K]: position evicted from that slot, -1 if empty  */
  int32_t n_ring;      /* selected rows read from the recent ring           */
} orc_step_info;

/* Replacement policies.  LRU: the slot with the oldest last-use step, ties to
 * the lowest slot.  Circular: a hand moves over the slots and takes the next
 * one not used in the current step.  Clock: hits and fills set a slot's
 * reference bit; the hand skips slots used in the current step, clears and
 * skips set bits, and takes the first slot with a clear bit.  Both hands
 * start at slot 0 and stop just past their last victim. */
#define ORC_LRU      0
#define ORC_CIRCULAR 1
#define ORC_CLOCK    2

orc_cache* orc_cache_new(int32_t C, int64_t hcap);   /* LRU */
orc_cache* orc_cache_new_policy(int32_t C, int64_t hcap, int32_t policy);
void       orc_cache_free(orc_cache* c);

/* Step t for a selection sel[0..K) (distinct positions < hcap, ascending):
 * positions the ring holds are left out; of the rest, hits first (last = t),
 * then each miss in order takes the slot minimising (last, slot) among slots
 * with last != t, evicting its position, and copies the 656-B host row into
 * the slot.  ring and info may be NULL.  Returns 0 or -1. */
int orc_cache_step(orc_cache* c, int32_t t, const int32_t* sel, int32_t K,
                   const uint8_t* host_rows, const orc_ring* ring, orc_step_info* info);

/* Reads every selected row from the ring if it holds it, else from its hot
 * slot, and dequantises it: out[i][0..576).  Returns -1 if a selected
 * position is in neither. */
int orc_gather(const orc_cache* c, const orc_ring* ring, const int32_t* sel, int32_t K,
               uint16_t* out);

/* State views (read-only, owned by the cache). */
const int32_t* orc_cache_slot_of(const orc_cache* c);  /* [hcap] pos -> slot  */
const int32_t* orc_cache_pos_of(const orc_cache* c);   /* [C] slot -> pos     */
const int32_t* orc_cache_last(const orc_cache* c);     /* [C] last-use step   */
const uint8_t* orc_cache_hot(const orc_cache* c);      /* [C][656] slot bytes */
const uint8_t* orc_cache_ref(const orc_cache* c);      /* [C] clock reference bits */
int32_t        orc_cache_hand(const orc_cache* c);     /* circular / clock hand */

/* Whole decode round for S sessions x L layers with a selection per group of R
 * layers (G = ceil(L/R)) and Q query rows per round (MTP verification: the
 * page's section "GPU cache management has hazards too"), units processed on
 * up to nthreads threads.  Every query selects its own top-K over the same
 * history; the cache step of each layer runs once on the ascending union of
 * the group's Q selections (so a position several queries select is one hit,
 * or one miss with one victim); each query's rows are gathered in its own
 * selection order.
 *   caches[s*L + l], host_rows[s*L + l], rings[s*L + l] (rings may be NULL)
 *   scores[(s*G + g)*Q + q] -> that query's fp32 scores, hist_len[s]
 *   sel_out [S*G*Q*K], out [S*L*Q*K*576] (NULL: skip the gather),
 *   infos[s*L + l] (NULL: none), each with Q*K entries per array: the union's
 *   entries first, -1 past the union.  Returns 0, or the first failing unit's
 *   -1. */
int orc_model_step(orc_cache* const* caches, const uint8_t* const* host_rows,
                   orc_ring* const* rings,
                   int32_t S, int32_t L, int32_t R, int32_t K, int32_t Q, int32_t t,
                   const float* const* scores, const int64_t* hist_len,
                   int32_t* sel_out, uint16_t* out, orc_step_info* infos,
                   int32_t nthreads);

#endif /* ORACLE_H */
