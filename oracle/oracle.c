/*
 * CPU oracle for heterogeneous batched LoRA over a paged memory pool.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the GPU library; it is plain C, fp64 throughout, slow on purpose.
 *
 * What it computes (one projection, every token t independently):
 *
 *   i      = adapter(t)            per segment for t < seg_offsets[S], per token after
 *   v[k]   = sum_{j < d_in}  x[t,j] * A_i[j,k]                      k < r_i
 *   y[t,n] = y0[t,n] + s_i * sum_{k < r_i} v[k] * B_i[k,n]          n < d_out
 *
 * and y[t,:] = y0[t,:] when i = -1 or r_i = 0.  Sources:
 *   - "Makale Bulteni - S-LoRA", section "Iddia ve Gerceklik: S-LoRA": a batched
 *     GEMM needs one weight for all rows; S-LoRA's kernel lets every token of a
 *     batch be multiplied by its own adapter matrix.
 *   - "S-LoRA: Serving Thousands of Concurrent LoRA Adapters" (paper review),
 *     section "Proposed method": base-model compute (batchable) is separate from
 *     adapter compute, so y0, the base output, is an input and only the adapter
 *     delta is added.
 *   - "S-LoRA: ..." overview (Chinese), sections "1. Unified Paging" and
 *     "2. Heterogeneous Batching": adapter weights of different ranks live in one
 *     paged pool with the KV cache and the kernels read non-contiguous memory.
 *   The LoRA product itself and s_i = alpha / r_i are the standard LoRA
 *   definition, which the pages name but do not print.
 *
 * Paged layout the oracle reads (its own convention; the pages give none):
 *   one page = page_elems consecutive elements; a row of length L occupies
 *   ceil(L / P) pages, the last one partially. For adapter i the page table holds,
 *   from entry base[i]: the r_i rows of A^T (row k = column k of A), ceil(d_in/P)
 *   entries each, then the r_i rows of B, ceil(d_out/P) entries each. Element j
 *   of A^T row k is pool[pt[base + k*cA + j/P] * P + j%P].
 *
 * Order of operations (fixed, so results are reproducible bit for bit): the
 * shrink sums ascending j, the expand sums ascending k, then y0 + s * acc.
 *
 * Decoders are written from the IEEE 754 binary16 and the bfloat16 bit layouts.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_E_INVALID (-1)

/* binary16: sign 1, exponent 5 (bias 15), fraction 10 */
double oracle_half_to_double(uint16_t h) {
  int sign = h >> 15;
  int ex = (h >> 10) & 0x1f;
  int fr = h & 0x3ff;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -24); /* subnormal: fr * 2^(1-15-10) */
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp((double)(fr | 0x400), ex - 25); /* (1024+fr) * 2^(ex-15-10) */
  return sign ? -v : v;
}

/* bfloat16: sign 1, exponent 8 (bias 127), fraction 7 */
double oracle_bfloat16_to_double(uint16_t b) {
  int sign = b >> 15;
  int ex = (b >> 7) & 0xff;
  int fr = b & 0x7f;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -133); /* subnormal: fr * 2^(1-127-7) */
  else if (ex == 255)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp((double)(fr | 0x80), ex - 134); /* (128+fr) * 2^(ex-127-7) */
  return sign ? -v : v;
}

typedef double (*decode_fn)(uint16_t);

/* Resolve which adapter token t uses. Returns -2 when the routing is invalid. */
static int32_t adapter_of(int64_t t, int32_t n_segments, const int32_t* seg_offsets,
                          const int32_t* seg_adapter, const int32_t* token_adapter) {
  int64_t seg_end = seg_offsets[n_segments];
  if (t < seg_end) {
    /* linear scan: the segment s with seg_offsets[s] <= t < seg_offsets[s+1] */
    for (int32_t s = 0; s < n_segments; ++s)
      if (t >= seg_offsets[s] && t < seg_offsets[s + 1]) return seg_adapter[s];
    return -2;
  }
  return token_adapter[t - seg_end];
}

typedef struct {
  decode_fn dec;
  int32_t d_in, d_out, P;
  int64_t n_tokens, n_pages;
  const uint16_t *x, *y0, *pool;
  const int32_t* pt;
  int64_t pt_len;
  int32_t n_adapters;
  const int64_t* base;
  const int32_t* rank;
  const double* scale;
  int32_t n_segments;
  const int32_t *seg_offsets, *seg_adapter, *token_adapter;
  const int64_t* eval_tokens;
  int64_t eval_begin, eval_end;
  double* y_ref;
  double* v_ref;
  int32_t r_max;
  int status;
} job;

/* Element e of row `row` of the block that starts at page-table entry `first`,
 * rows of length L, c pages per row. Returns NULL when out of range. */
static const uint16_t* paged_elem(const job* J, int64_t first, int32_t row, int32_t c, int32_t e) {
  int64_t entry = first + (int64_t)row * c + e / J->P;
  if (entry < 0 || entry >= J->pt_len) return NULL;
  int64_t page = J->pt[entry];
  if (page < 0 || page >= J->n_pages) return NULL;
  return J->pool + page * (int64_t)J->P + e % J->P;
}

static void* run_job(void* arg) {
  job* J = (job*)arg;
  const int32_t cA = (J->d_in + J->P - 1) / J->P;
  const int32_t cB = (J->d_out + J->P - 1) / J->P;
  double* v = (double*)malloc(sizeof(double) * (J->r_max > 0 ? J->r_max : 1));
  if (!v) { J->status = ORACLE_E_INVALID; return NULL; }
  for (int64_t q = J->eval_begin; q < J->eval_end; ++q) {
    int64_t t = J->eval_tokens ? J->eval_tokens[q] : q;
    double* yr = J->y_ref + q * (int64_t)J->d_out;
    if (t < 0 || t >= J->n_tokens) { J->status = ORACLE_E_INVALID; break; }
    int32_t i = adapter_of(t, J->n_segments, J->seg_offsets, J->seg_adapter, J->token_adapter);
    if (i < -1 || i >= J->n_adapters) { J->status = ORACLE_E_INVALID; break; }
    int32_t r = (i >= 0) ? J->rank[i] : 0;
    if (r < 0 || r > J->r_max) { J->status = ORACLE_E_INVALID; break; }
    const uint16_t* y0row = J->y0 + t * (int64_t)J->d_out;
    if (r == 0) {
      for (int32_t n = 0; n < J->d_out; ++n) yr[n] = J->dec(y0row[n]);
      if (J->v_ref)
        for (int32_t k = 0; k < J->r_max; ++k) J->v_ref[q * (int64_t)J->r_max + k] = 0.0;
      continue;
    }
    if (J->base[i] < 0) { J->status = ORACLE_E_INVALID; break; }
    const int64_t baseA = J->base[i];
    const int64_t baseB = J->base[i] + (int64_t)r * cA;
    const uint16_t* xrow = J->x + t * (int64_t)J->d_in;
    const double s = J->scale[i];
    /* shrink: v[k] = sum_j x[t,j] * A^T[k,j], ascending j */
    for (int32_t k = 0; k < r; ++k) {
      double acc = 0.0;
      for (int32_t j = 0; j < J->d_in; ++j) {
        const uint16_t* a = paged_elem(J, baseA, k, cA, j);
        if (!a) { J->status = ORACLE_E_INVALID; goto done; }
        acc += J->dec(xrow[j]) * J->dec(*a);
      }
      v[k] = acc;
    }
    if (J->v_ref) {
      for (int32_t k = 0; k < J->r_max; ++k)
        J->v_ref[q * (int64_t)J->r_max + k] = (k < r) ? v[k] : 0.0;
    }
    /* expand: y[t,n] = y0[t,n] + s * sum_k v[k] * B[k,n], ascending k */
    for (int32_t n = 0; n < J->d_out; ++n) {
      double acc = 0.0;
      for (int32_t k = 0; k < r; ++k) {
        const uint16_t* b = paged_elem(J, baseB, k, cB, n);
        if (!b) { J->status = ORACLE_E_INVALID; goto done; }
        acc += v[k] * J->dec(*b);
      }
      yr[n] = J->dec(y0row[n]) + s * acc;
    }
  }
done:
  free(v);
  return NULL;
}

/*
 * y_ref[q, :] for q < n_eval, token t = eval_tokens[q] (or q when eval_tokens is
 * NULL, then n_eval must equal n_tokens). v_ref (optional) gets v[q, k], zero for
 * k >= rank. dtype: 0 = fp16, 1 = bf16 (x, y0 and pool all of that type, as
 * uint16 bit patterns). Returns 0, or -1 for invalid routing, page-table or pool
 * indices (every index is checked before it is used).
 */
int oracle_lora(int32_t dtype, int32_t d_in, int32_t d_out, int64_t n_tokens,
                const uint16_t* x, const uint16_t* y0, const uint16_t* pool, int64_t n_pages,
                int32_t page_elems, const int32_t* page_table, int64_t pt_len,
                int32_t n_adapters, const int64_t* base, const int32_t* rank,
                const double* scale, int32_t n_segments, const int32_t* seg_offsets,
                const int32_t* seg_adapter, const int32_t* token_adapter, int64_t n_eval,
                const int64_t* eval_tokens, double* y_ref, double* v_ref, int32_t r_max,
                int32_t n_threads) {
  if (dtype != 0 && dtype != 1) return ORACLE_E_INVALID;
  if (d_in <= 0 || d_out <= 0 || page_elems <= 0 || n_tokens < 0 || n_eval < 0) return ORACLE_E_INVALID;
  if (n_segments < 0 || !seg_offsets || seg_offsets[0] != 0) return ORACLE_E_INVALID;
  for (int32_t s = 0; s < n_segments; ++s)
    if (seg_offsets[s + 1] < seg_offsets[s]) return ORACLE_E_INVALID;
  if (seg_offsets[n_segments] > n_tokens) return ORACLE_E_INVALID;
  if (!eval_tokens && n_eval != n_tokens) return ORACLE_E_INVALID;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if (n_eval == 0) return ORACLE_OK;
  if ((int64_t)n_threads > n_eval) n_threads = (int32_t)n_eval;

  job proto;
  memset(&proto, 0, sizeof proto);
  proto.dec = dtype == 0 ? oracle_half_to_double : oracle_bfloat16_to_double;
  proto.d_in = d_in; proto.d_out = d_out; proto.P = page_elems;
  proto.n_tokens = n_tokens; proto.n_pages = n_pages;
  proto.x = x; proto.y0 = y0; proto.pool = pool;
  proto.pt = page_table; proto.pt_len = pt_len;
  proto.n_adapters = n_adapters; proto.base = base; proto.rank = rank; proto.scale = scale;
  proto.n_segments = n_segments; proto.seg_offsets = seg_offsets;
  proto.seg_adapter = seg_adapter; proto.token_adapter = token_adapter;
  proto.eval_tokens = eval_tokens; proto.y_ref = y_ref; proto.v_ref = v_ref; proto.r_max = r_max;

  job* jobs = (job*)calloc((size_t)n_threads, sizeof(job));
  pthread_t* th = (pthread_t*)calloc((size_t)n_threads, sizeof(pthread_t));
  int* started = (int*)calloc((size_t)n_threads, sizeof(int));
  if (!jobs || !th || !started) { free(jobs); free(th); free(started); return ORACLE_E_INVALID; }
  for (int32_t w = 0; w < n_threads; ++w) {
    jobs[w] = proto;
    jobs[w].eval_begin = n_eval * w / n_threads;
    jobs[w].eval_end = n_eval * (w + 1) / n_threads;
  }
  for (int32_t w = 1; w < n_threads; ++w)
    started[w] = pthread_create(&th[w], NULL, run_job, &jobs[w]) == 0;
  run_job(&jobs[0]);
  int status = jobs[0].status;
  for (int32_t w = 1; w < n_threads; ++w) {
    if (started[w]) pthread_join(th[w], NULL);
    else run_job(&jobs[w]);
    if (jobs[w].status) status = jobs[w].status;
  }
  free(jobs); free(th); free(started);
  return status;
}
