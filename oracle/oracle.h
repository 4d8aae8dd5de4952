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
 * patterns (non-finite scales included; NaN results are 0x7FC0 | sign). */
void orc_dequant_table(uint16_t* table);

/* LRU hot cache of one (session, layer). */
typedef struct orc_cache orc_cache;

typedef struct orc_step_info {
  int32_t n_hit, n_miss, n_evict;
  int32_t* slot;       /* [K]: slot of sel[i] after the step                 */
  int32_t* miss_pos;   /* [K]: misses in processing order (ascending pos)    */
  int32_t* victim;     /* [K]: slot given to miss i                          */
  int32_t* evicted;    /* [K]: position evicted from that slot, -1 if empty  */
} orc_step_info;

orc_cache* orc_cache_new(int32_t C, int64_t hcap);
void       orc_cache_free(orc_cache* c);

/* Step t for a selection sel[0..K) (distinct positions < hcap, ascending):
 * hits first (last = t), then each miss in order takes the slot minimising
 * (last, slot) among slots with last != t, evicting its position, and copies
 * the 656-B host row into the slot.  info may be NULL.  Returns 0 or -1. */
int orc_cache_step(orc_cache* c, int32_t t, const int32_t* sel, int32_t K,
                   const uint8_t* host_rows, orc_step_info* info);

/* Reads every selected row from its hot slot and dequantises it:
 * out[i][0..576).  Returns -1 if a selected position is not resident. */
int orc_gather(const orc_cache* c, const int32_t* sel, int32_t K, uint16_t* out);

/* State views (read-only, owned by the cache). */
const int32_t* orc_cache_slot_of(const orc_cache* c);  /* [hcap] pos -> slot  */
const int32_t* orc_cache_pos_of(const orc_cache* c);   /* [C] slot -> pos     */
const int32_t* orc_cache_last(const orc_cache* c);     /* [C] last-use step   */
const uint8_t* orc_cache_hot(const orc_cache* c);      /* [C][656] slot bytes */

/* Whole decode step for S sessions x L layers with a selection per group of R
 * layers (G = ceil(L/R)), units processed on up to nthreads threads.
 *   caches[s*L + l], host_rows[s*L + l]
 *   scores[s*G + g] -> that unit's fp32 scores, hist_len[s]
 *   sel_out [S*G*K], out [S*L*K*576] (NULL: skip the gather),
 *   infos[s*L + l] (NULL: none).  Returns 0, or the first failing unit's -1. */
int orc_model_step(orc_cache* const* caches, const uint8_t* const* host_rows,
                   int32_t S, int32_t L, int32_t R, int32_t K, int32_t t,
                   const float* const* scores, const int64_t* hist_len,
                   int32_t* sel_out, uint16_t* out, orc_step_info* infos,
                   int32_t nthreads);

#endif /* ORACLE_H */
