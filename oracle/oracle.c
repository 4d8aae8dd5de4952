/*
 * oracle.c — plain CPU oracle of the sparse-KV hot-cache decode step.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product path.  Written from
 * the page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading"
 * (zhuai.tech), sections "Separate historical capacity from the current
 * working set", "Decision three: let the GPU manage the hot cache directly"
 * and "GPU cache management has hazards too".  Each function is the plain
 * definition of its step, in the order the step is defined; no blocking,
 * fusion or reordering.  Parity pins: tests/test_oracle_*.py.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- top-K -- */

/* IEEE-754 totalOrder as an unsigned integer: negative numbers reverse their
 * bit order below all positive ones, so -0 < +0 and NaNs sort by their bits. */
static uint32_t total_order_key(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

typedef struct { uint32_t key; int32_t pos; } ranked;

/* Rank order: larger key first; equal keys by ascending position. */
static int cmp_rank(const void* a, const void* b) {
  const ranked* x = (const ranked*)a;
  const ranked* y = (const ranked*)b;
  if (x->key != y->key) return x->key > y->key ? -1 : 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_int32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int orc_topk(const float* scores, int64_t H, int32_t K, int32_t* sel) {
  if (K < 1 || (int64_t)K > H) return -1;
  ranked* all = (ranked*)malloc((size_t)H * sizeof(ranked));
  if (!all) return -1;
  for (int64_t p = 0; p < H; ++p) {
    all[p].key = total_order_key(scores[p]);
    all[p].pos = (int32_t)p;
  }
  /* Full sort of every position by rank, then the first K by position. */
  qsort(all, (size_t)H, sizeof(ranked), cmp_rank);
  for (int32_t i = 0; i < K; ++i) sel[i] = all[i].pos;
  qsort(sel, (size_t)K, sizeof(int32_t), cmp_int32);
  free(all);
  return 0;
}

/* -------------------------------------------------------------- dequant -- */

/* Value of an IEEE binary16 bit pattern (sign, 5-bit exponent, 10-bit
 * fraction; exponent 0 = subnormal, 31 = Inf/NaN). */
static double fp16_value(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);            /* 0.m x 2^-14 = m x 2^-24        */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* 1.m x 2^(e-15)                */
  return sign ? -v : v;
}

/* Round a double to the nearest bfloat16 (1 sign, 8 exponent, 7 fraction
 * bits), ties to even, and return its bit pattern. */
static uint16_t bf16_round_double(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7FC0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  double m = frexp(a, &e);            /* a = m x 2^e, m in [0.5, 1)        */
  int E = e - 1;                      /* a = (2m) x 2^E, 2m in [1, 2)      */
  double units, ulp_exp;
  if (E >= -126) {
    units = ldexp(m, 8);              /* significand in units of its ulp   */
    ulp_exp = E - 7;
  } else {                            /* subnormal: fixed ulp 2^-133       */
    units = ldexp(a, 133);
    ulp_exp = -133;
  }
  double fl = floor(units), frac = units - fl;
  if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  double r = ldexp(fl, (int)ulp_exp); /* rounded magnitude, exact          */
  if (r >= 0x1.0p128) return sign | 0x7F80;  /* beyond the bf16 range     */
  /* Encode r: normal if r >= 2^-126, else subnormal with ulp 2^-133. */
  if (r < 0x1.0p-126) return sign | (uint16_t)ldexp(r, 133);
  int re;
  double rm = frexp(r, &re);          /* r = rm x 2^re, rm in [0.5, 1)     */
  uint16_t exp_field = (uint16_t)(re - 1 + 127);
  uint16_t frac_field = (uint16_t)(ldexp(rm, 8) - 128.0);
  return sign | (uint16_t)(exp_field << 7) | frac_field;
}

uint16_t orc_dequant_elem(int8_t q, uint16_t scale_bits) {
  /* |q| <= 2^7 and an fp16 significand has 11 bits: the product is exact in
   * double (and in fp32), so the only rounding is the one to bf16. */
  return bf16_round_double((double)q * fp16_value(scale_bits));
}

void orc_dequant_row(const uint8_t* row, uint16_t* out) {
  for (int j = 0; j < 512; ++j) {
    int g = j / 64;
    uint16_t scale = (uint16_t)(row[512 + 2 * g] | (row[512 + 2 * g + 1] << 8));
    out[j] = orc_dequant_elem((int8_t)row[j], scale);
  }
  for (int k = 0; k < 64; ++k)
    out[512 + k] = (uint16_t)(row[528 + 2 * k] | (row[528 + 2 * k + 1] << 8));
}

void orc_dequant_table(uint16_t* table) {
  for (int q = -128; q < 128; ++q)
    for (int s = 0; s < 65536; ++s)
      table[(size_t)(q + 128) * 65536 + s] = orc_dequant_elem((int8_t)q, (uint16_t)s);
}

/* ---------------------------------------------------------- recent ring -- */

/* New rows of one (session, layer) (page "From 1M Total to 15+ × 1M Contexts:
 * GLM-5.3 KV Cache Offloading", data-flow figure of "Decision three" and
 * section "GPU cache management has hazards too"): a row appended on the GPU
 * first lives in a recent ring that holds the last `rows` appended rows; it
 * reaches host RAM only through a batched copyback.  Here the ring copies
 * every complete batch of `batch` rows not yet in host RAM as soon as the
 * batch is complete, and a flush copies whatever is left (section "Capacity
 * optimization must survive the session lifecycle"). */
struct orc_ring {
  int32_t rows, batch;
  int64_t first;     /* first appended position, -1 before the first append */
  int64_t end;       /* one past the last appended position                */
  int64_t copied;    /* appended rows [first, copied) are in host RAM      */
  int64_t* pos;      /* ring entry -> position it holds, -1 if none        */
  uint8_t* data;     /* ring entry -> row bytes                            */
};

orc_ring* orc_ring_new(int32_t rows, int32_t batch) {
  if (rows < 1 || batch < 1 || batch > rows) return NULL;
  orc_ring* r = (orc_ring*)calloc(1, sizeof *r);
  if (!r) return NULL;
  r->rows = rows;
  r->batch = batch;
  r->first = r->end = r->copied = -1;
  r->pos = (int64_t*)malloc((size_t)rows * sizeof(int64_t));
  r->data = (uint8_t*)calloc((size_t)rows, ORC_ROW_BYTES);
  if (!r->pos || !r->data) {
    orc_ring_free(r);
    return NULL;
  }
  for (int32_t i = 0; i < rows; ++i) r->pos[i] = -1;
  return r;
}

void orc_ring_free(orc_ring* r) {
  if (!r) return;
  free(r->pos);
  free(r->data);
  free(r);
}

/* Copies the appended rows not yet in host RAM out of the ring. */
static void ring_copy_back(orc_ring* r, uint8_t* host_rows) {
  for (int64_t p = r->copied; p < r->end; ++p) {
    const int32_t e = (int32_t)(p % r->rows);
    memcpy(host_rows + (size_t)p * ORC_ROW_BYTES, r->data + (size_t)e * ORC_ROW_BYTES,
           ORC_ROW_BYTES);
  }
  r->copied = r->end;
}

int orc_ring_append(orc_ring* r, int64_t p, const uint8_t* row, uint8_t* host_rows) {
  if (p < 0 || (r->first >= 0 && p != r->end)) return -1;
  if (r->first < 0) r->first = r->end = r->copied = p;
  const int32_t e = (int32_t)(p % r->rows);
  /* the entry's previous row must already be in host RAM */
  if (r->pos[e] >= 0 && r->pos[e] >= r->copied) return -1;
  memcpy(r->data + (size_t)e * ORC_ROW_BYTES, row, ORC_ROW_BYTES);
  r->pos[e] = p;
  r->end = p + 1;
  if (r->end - r->copied >= r->batch) ring_copy_back(r, host_rows);
  return 0;
}

int64_t orc_ring_flush(orc_ring* r, uint8_t* host_rows) {
  if (r->first < 0) return 0;
  ring_copy_back(r, host_rows);
  return r->copied;
}

const uint8_t* orc_ring_row(const orc_ring* r, int64_t p) {
  if (!r || p < 0) return NULL;
  const int32_t e = (int32_t)(p % r->rows);
  return r->pos[e] == p ? r->data + (size_t)e * ORC_ROW_BYTES : NULL;
}

int64_t orc_ring_copied(const orc_ring* r) { return r->first < 0 ? 0 : r->copied; }

/* ------------------------------------------------------------ attention -- */

/* Value of a bfloat16 bit pattern (the upper half of an IEEE binary32). */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* MLA decode attention over K gathered rows, in double precision.  For each
 * head h: z_i = scale * sum over all 576 values of q[h] * row_i, weights =
 * softmax(z) (largest score subtracted first), out[h][d] = sum_i w_i *
 * row_i[d] for the 512 latent values. */
void orc_attend(const uint16_t* q, const uint16_t* rows, int32_t H, int32_t K, double scale,
                double* out) {
  double* z = (double*)malloc((size_t)K * sizeof(double));
  if (!z) return;
  for (int32_t h = 0; h < H; ++h) {
    const uint16_t* qh = q + (size_t)h * ORC_OUT_ELEMS;
    double zmax = -INFINITY;
    for (int32_t i = 0; i < K; ++i) {
      const uint16_t* x = rows + (size_t)i * ORC_OUT_ELEMS;
      double acc = 0.0;
      for (int d = 0; d < ORC_OUT_ELEMS; ++d) acc += bf16_value(qh[d]) * bf16_value(x[d]);
      z[i] = scale * acc;
      if (z[i] > zmax) zmax = z[i];
    }
    double sum = 0.0;
    for (int32_t i = 0; i < K; ++i) {
      z[i] = exp(z[i] - zmax);
      sum += z[i];
    }
    double* oh = out + (size_t)h * 512;
    for (int d = 0; d < 512; ++d) oh[d] = 0.0;
    for (int32_t i = 0; i < K; ++i) {
      const uint16_t* x = rows + (size_t)i * ORC_OUT_ELEMS;
      const double w = z[i] / sum;
      for (int d = 0; d < 512; ++d) oh[d] += w * bf16_value(x[d]);
    }
  }
  free(z);
}

/* ------------------------------------------------------------ LRU cache -- */

struct orc_cache {
  int32_t C;
  int64_t hcap;
  int32_t* slot_of;  /* position -> slot, -1 if not resident */
  int32_t* pos_of;   /* slot -> position, -1 if empty        */
  int32_t* last;     /* slot -> last-use step, -1 if unused  */
  uint8_t* hot;      /* slot contents                        */
  int32_t policy;    /* ORC_LRU, ORC_CIRCULAR or ORC_CLOCK    */
  int32_t hand;      /* circular / clock hand                 */
  uint8_t* ref;      /* clock reference bits                  */
};

orc_cache* orc_cache_new(int32_t C, int64_t hcap) { return orc_cache_new_policy(C, hcap, ORC_LRU); }

orc_cache* orc_cache_new_policy(int32_t C, int64_t hcap, int32_t policy) {
  if (C < 1 || hcap < 1 || policy < ORC_LRU || policy > ORC_CLOCK) return NULL;
  orc_cache* c = (orc_cache*)calloc(1, sizeof *c);
  if (!c) return NULL;
  c->C = C;
  c->hcap = hcap;
  c->slot_of = (int32_t*)malloc((size_t)hcap * sizeof(int32_t));
  c->pos_of = (int32_t*)malloc((size_t)C * sizeof(int32_t));
  c->last = (int32_t*)malloc((size_t)C * sizeof(int32_t));
  c->hot = (uint8_t*)calloc((size_t)C, ORC_ROW_BYTES);
  c->ref = (uint8_t*)calloc((size_t)C, 1);
  c->policy = policy;
  c->hand = 0;
  if (!c->slot_of || !c->pos_of || !c->last || !c->hot || !c->ref) {
    orc_cache_free(c);
    return NULL;
  }
  for (int64_t p = 0; p < hcap; ++p) c->slot_of[p] = -1;
  for (int32_t v = 0; v < C; ++v) c->pos_of[v] = -1, c->last[v] = -1;
  return c;
}

void orc_cache_free(orc_cache* c) {
  if (!c) return;
  free(c->slot_of);
  free(c->pos_of);
  free(c->last);
  free(c->hot);
  free(c->ref);
  free(c);
}

/* The slot minimising (last, slot) over slots not used in step t. */
static int32_t lru_victim(const orc_cache* c, int32_t t) {
  int32_t best = -1;
  for (int32_t v = 0; v < c->C; ++v) {
    if (c->last[v] == t) continue;
    if (best < 0 || c->last[v] < c->last[best]) best = v;
  }
  return best;
}

/* Circular eviction that skips pinned slots (page "From 1M Total to 15+ × 1M
 * Contexts: GLM-5.3 KV Cache Offloading", section "GPU cache management has
 * hazards too"): the hand moves to the next slot not used in step t, which is
 * the victim, and passes it. */
static int32_t circular_victim(orc_cache* c, int32_t t) {
  for (int32_t n = 0; n < c->C; ++n) {
    int32_t v = c->hand;
    c->hand = (c->hand + 1) % c->C;
    if (c->last[v] != t) return v;
  }
  return -1;
}

/* Clock with reference bits (same section): the hand skips slots used in step
 * t, clears and skips slots whose reference bit is set, and takes the first
 * slot whose bit is clear.  Two revolutions always suffice. */
static int32_t clock_victim(orc_cache* c, int32_t t) {
  for (int32_t n = 0; n < 2 * c->C; ++n) {
    int32_t v = c->hand;
    c->hand = (c->hand + 1) % c->C;
    if (c->last[v] == t) continue;
    if (c->ref[v]) {
      c->ref[v] = 0;
      continue;
    }
    return v;
  }
  return -1;
}

int orc_cache_step(orc_cache* c, int32_t t, const int32_t* sel, int32_t K,
                   const uint8_t* host_rows, const orc_ring* ring, orc_step_info* info) {
  if (K < 1 || K > c->C) return -1;
  for (int32_t i = 0; i < K; ++i)
    if (sel[i] < 0 || sel[i] >= c->hcap) return -1;
  int32_t n_hit = 0, n_miss = 0, n_evict = 0, n_ring = 0;
  /* Rows still in the recent ring are read from there and leave the cache
   * alone. */
  for (int32_t i = 0; i < K; ++i) n_ring += orc_ring_row(ring, sel[i]) != NULL;
  /* Hits: a selected position already resident is used in step t. */
  for (int32_t i = 0; i < K; ++i) {
    if (orc_ring_row(ring, sel[i])) continue;
    int32_t s = c->slot_of[sel[i]];
    if (s >= 0) {
      c->last[s] = t;
      ++n_hit;
      c->ref[s] = 1;
    }
  }
  /* Misses, one at a time in selection order. */
  for (int32_t i = 0; i < K; ++i) {
    int32_t p = sel[i];
    if (orc_ring_row(ring, p) || c->slot_of[p] >= 0) continue;
    int32_t v = c->policy == ORC_CIRCULAR ? circular_victim(c, t)
              : c->policy == ORC_CLOCK    ? clock_victim(c, t)
                                          : lru_victim(c, t);
    if (v < 0) return -1;
    int32_t old = c->pos_of[v];
    if (old >= 0) {
      c->slot_of[old] = -1;
      ++n_evict;
    }
    c->pos_of[v] = p;
    c->slot_of[p] = v;
    c->last[v] = t;
    c->ref[v] = 1;
    memcpy(c->hot + (size_t)v * ORC_ROW_BYTES, host_rows + (size_t)p * ORC_ROW_BYTES,
           ORC_ROW_BYTES);
    if (info) {
      info->miss_pos[n_miss] = p;
      info->victim[n_miss] = v;
      info->evicted[n_miss] = old;
    }
    ++n_miss;
  }
  if (info) {
    for (int32_t i = 0; i < K; ++i)
      info->slot[i] = orc_ring_row(ring, sel[i]) ? c->C + (int32_t)(sel[i] % ring->rows)
                                                 : c->slot_of[sel[i]];
    for (int32_t j = n_miss; j < K; ++j)
      info->miss_pos[j] = info->victim[j] = info->evicted[j] = -1;
    info->n_hit = n_hit;
    info->n_miss = n_miss;
    info->n_evict = n_evict;
    info->n_ring = n_ring;
  }
  return 0;
}

int orc_gather(const orc_cache* c, const orc_ring* ring, const int32_t* sel, int32_t K,
               uint16_t* out) {
  for (int32_t i = 0; i < K; ++i) {
    if (sel[i] < 0 || sel[i] >= c->hcap) return -1;
    const uint8_t* rrow = orc_ring_row(ring, sel[i]);
    if (rrow) {
      orc_dequant_row(rrow, out + (size_t)i * ORC_OUT_ELEMS);
      continue;
    }
    int32_t s = c->slot_of[sel[i]];
    if (s < 0) return -1;
    orc_dequant_row(c->hot + (size_t)s * ORC_ROW_BYTES, out + (size_t)i * ORC_OUT_ELEMS);
  }
  return 0;
}

const int32_t* orc_cache_slot_of(const orc_cache* c) { return c->slot_of; }
const int32_t* orc_cache_pos_of(const orc_cache* c) { return c->pos_of; }
const int32_t* orc_cache_last(const orc_cache* c) { return c->last; }
const uint8_t* orc_cache_hot(const orc_cache* c) { return c->hot; }
const uint8_t* orc_cache_ref(const orc_cache* c) { return c->ref; }
int32_t orc_cache_hand(const orc_cache* c) { return c->hand; }

/* --------------------------------------------------- whole-model driver -- */

typedef struct {
  orc_cache* const* caches;
  const uint8_t* const* host_rows;
  orc_ring* const* rings;
  int32_t S, L, R, K, G, Q, t;
  const float* const* scores;
  const int64_t* hist_len;
  int32_t* sel_out;
  uint16_t* out;
  orc_step_info* infos;
  pthread_mutex_t lock;
  int32_t next_unit;
  int status;
} model_job;

/* One selection unit (session s, group g) of a round: every query's top-K,
 * the ascending union of the Q selections, one cache step on the union for
 * each layer of the group, then each query's rows gathered in its own order. */
static int run_unit(model_job* j, int32_t u) {
  int32_t s = u / j->G, g = u % j->G;
  const int32_t QK = j->Q * j->K;
  int32_t* sel = j->sel_out + (size_t)u * QK;     /* [Q][K] */
  for (int32_t q = 0; q < j->Q; ++q)
    if (orc_topk(j->scores[(size_t)u * j->Q + q], j->hist_len[s], j->K, sel + (size_t)q * j->K))
      return -1;
  int32_t* uni = (int32_t*)malloc((size_t)QK * sizeof(int32_t));
  if (!uni) return -1;
  memcpy(uni, sel, (size_t)QK * sizeof(int32_t));
  qsort(uni, (size_t)QK, sizeof(int32_t), cmp_int32);
  int32_t n = 0;
  for (int32_t i = 0; i < QK; ++i)
    if (n == 0 || uni[i] != uni[n - 1]) uni[n++] = uni[i];
  int status = 0;
  int32_t l_end = (g + 1) * j->R < j->L ? (g + 1) * j->R : j->L;
  for (int32_t l = g * j->R; l < l_end && !status; ++l) {
    size_t sl = (size_t)s * j->L + l;
    orc_step_info* info = j->infos ? &j->infos[sl] : NULL;
    const orc_ring* ring = j->rings ? j->rings[sl] : NULL;
    if (orc_cache_step(j->caches[sl], j->t, uni, n, j->host_rows[sl], ring, info)) {
      status = -1;
      break;
    }
    if (info)
      for (int32_t i = n; i < QK; ++i)
        info->slot[i] = info->miss_pos[i] = info->victim[i] = info->evicted[i] = -1;
    for (int32_t q = 0; q < j->Q && j->out; ++q)
      if (orc_gather(j->caches[sl], ring, sel + (size_t)q * j->K, j->K,
                     j->out + (sl * j->Q + q) * (size_t)j->K * ORC_OUT_ELEMS))
        status = -1;
  }
  free(uni);
  return status;
}

static void* model_worker(void* arg) {
  model_job* j = (model_job*)arg;
  for (;;) {
    pthread_mutex_lock(&j->lock);
    int32_t u = j->next_unit++;
    pthread_mutex_unlock(&j->lock);
    if (u >= j->S * j->G) break;
    if (run_unit(j, u)) {
      pthread_mutex_lock(&j->lock);
      j->status = -1;
      pthread_mutex_unlock(&j->lock);
    }
  }
  return NULL;
}

int orc_model_step(orc_cache* const* caches, const uint8_t* const* host_rows,
                   orc_ring* const* rings,
                   int32_t S, int32_t L, int32_t R, int32_t K, int32_t Q, int32_t t,
                   const float* const* scores, const int64_t* hist_len,
                   int32_t* sel_out, uint16_t* out, orc_step_info* infos,
                   int32_t nthreads) {
  if (S < 1 || L < 1 || R < 1 || K < 1 || Q < 1) return -1;
  model_job j;
  j.caches = caches;
  j.host_rows = host_rows;
  j.rings = rings;
  j.S = S, j.L = L, j.R = R, j.K = K, j.G = (L + R - 1) / R, j.Q = Q, j.t = t;
  j.scores = scores;
  j.hist_len = hist_len;
  j.sel_out = sel_out;
  j.out = out;
  j.infos = infos;
  j.next_unit = 0;
  j.status = 0;
  pthread_mutex_init(&j.lock, NULL);
  int32_t units = S * j.G;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = units;
  if (nthreads == 1) {
    model_worker(&j);
  } else {
    pthread_t* th = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
    int32_t started = 0;
    for (; th && started < nthreads; ++started)
      if (pthread_create(&th[started], NULL, model_worker, &j)) break;
    if (started == 0) model_worker(&j);
    for (int32_t i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&j.lock);
  return j.status;
}
