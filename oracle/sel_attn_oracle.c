/*
 * CPU oracle for prompt-phase selection attention over INT8 paged K/V.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing outside tests/, the package's smoke check
 * and the benchmark's CPU-baseline leg may load or call this library; the HIP
 * path shares no code, header, table or helper with it.
 *
 * Page cited: #2808 "sycl: prompt attention over 8-query selection unions on
 * XMX (opt-in STRATA_PROMPT_ATTN_UNION=1)".
 *
 * What is computed, as the page defines it:
 *   - Union (section Summary): one sorted list per group of 8 adjacent query
 *     positions holding every cell any of them selected, each entry carrying
 *     the set of group positions that selected it. Section Extra Notes: a cell is an int32 and its
 *     8-position mask a separate byte. Bit i of the mask is position 8g+i.
 *   - Attention (section Summary): every position attends to exactly the cells
 *     it selected, as the per-position FP32 kernel does; cells of pages that are
 *     not resident are masked (section Extra Notes, "Not tested" item; the
 *     accuracy list in section Summary includes non-resident pages in the
 *     parity self-test). INT8 K/V are
 *     dequantised with per-cell, per-KV-head scales. Query head h reads KV head
 *     h / q_per_kv. The softmax runs over the position's own set only.
 *
 * This is the plain definition, written out: a per-position gather of the
 * position's deduplicated resident cells, scores, a softmax and a weighted sum,
 * all in double precision. Duplicate entries in a selection row count once
 * (set semantics). A position with no resident selected cell outputs zeros.
 *
 * Layouts (row-major):
 *   sel          int32 [n_q][sel_cap]          sel_len int32 [n_q]
 *   k/v_pool     int8  [n_pages][n_kv][page_size][head_dim]
 *   k/v_scale    float [n_pages][n_kv][page_size]
 *   page_table   int32 [ceil(n_ctx/page_size)]  (-1 = not resident)
 *   q            float [n_q][n_kv*q_per_kv][head_dim]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* The set of cells in one selection row: copy, sort ascending, drop repeats.
 * Returns the set size, or -1 if a cell lies outside [0, n_ctx). */
static int row_as_set(const int32_t* row, int len, int n_ctx, int32_t* out) {
  for (int e = 0; e < len; ++e) {
    if (row[e] < 0 || row[e] >= n_ctx) return -1;
    out[e] = row[e];
  }
  qsort(out, (size_t)len, sizeof(int32_t), cmp_i32);
  int n = 0;
  for (int e = 0; e < len; ++e)
    if (n == 0 || out[n - 1] != out[e]) out[n++] = out[e];
  return n;
}

static int contains(const int32_t* set, int n, int32_t c) {
  int lo = 0, hi = n - 1;
  while (lo <= hi) {
    int mid = lo + (hi - lo) / 2;
    if (set[mid] == c) return 1;
    if (set[mid] < c) lo = mid + 1; else hi = mid - 1;
  }
  return 0;
}

/*
 * Union of every group of 8 consecutive query indices [8g, 8g+8) ∩ [0, n_q).
 * union_cells/union_mask have room for 8*sel_cap entries per group.
 * Returns ORACLE_OK, or ORACLE_EINVAL for a bad sel_len or cell.
 */
int oracle_union(int n_q, int sel_cap, int n_ctx, const int32_t* sel,
                 const int32_t* sel_len, int32_t* union_cells,
                 uint8_t* union_mask, int32_t* union_len) {
  if (n_q < 0 || sel_cap < 1 || n_ctx < 1) return ORACLE_EINVAL;
  const int n_groups = (n_q + 7) / 8;
  const long ucap = 8L * sel_cap;
  int err = ORACLE_OK;
  #pragma omp parallel for schedule(dynamic, 4)
  for (int g = 0; g < n_groups; ++g) {
    int32_t* sets = (int32_t*)malloc(sizeof(int32_t) * (size_t)ucap);
    int32_t* all = (int32_t*)malloc(sizeof(int32_t) * (size_t)ucap);
    int set_n[8], set_off[8], n_all = 0, bad = 0;
    const int n_pos = (n_q - 8 * g) < 8 ? (n_q - 8 * g) : 8;
    if (!sets || !all) { bad = ORACLE_ENOMEM; goto done; }
    for (int i = 0; i < n_pos; ++i) {
      const int j = 8 * g + i;
      const int len = sel_len[j];
      if (len < 0 || len > sel_cap) { bad = ORACLE_EINVAL; goto done; }
      set_off[i] = i * sel_cap;
      set_n[i] = row_as_set(sel + (size_t)j * sel_cap, len, n_ctx, sets + set_off[i]);
      if (set_n[i] < 0) { bad = ORACLE_EINVAL; goto done; }
      memcpy(all + n_all, sets + set_off[i], sizeof(int32_t) * (size_t)set_n[i]);
      n_all += set_n[i];
    }
    /* sorted set union of the group's rows */
    qsort(all, (size_t)n_all, sizeof(int32_t), cmp_i32);
    int n_u = 0;
    for (int e = 0; e < n_all; ++e)
      if (n_u == 0 || all[n_u - 1] != all[e]) all[n_u++] = all[e];
    /* the chooser byte of each union cell: one bit per group position that selected it */
    for (int u = 0; u < n_u; ++u) {
      uint8_t m = 0;
      for (int i = 0; i < n_pos; ++i)
        if (contains(sets + set_off[i], set_n[i], all[u])) m |= (uint8_t)(1u << i);
      union_cells[(size_t)g * ucap + u] = all[u];
      union_mask[(size_t)g * ucap + u] = m;
    }
    union_len[g] = n_u;
  done:
    if (bad) {
      #pragma omp critical
      err = bad;
    }
    free(sets);
    free(all);
  }
  return err;
}

/*
 * Attention output of the query indices listed in rows[0..n_rows) (all n_q in
 * order when rows is NULL), in double precision:
 *   R_j      = { c in set(sel[j]) : page_table[c / page_size] >= 0 }
 *   k_c, v_c = int8 row * its fp32 scale, promoted to double
 *   s_c      = softmax_scale * <q[j][h], k_c>          for c in R_j
 *   out[r][h] = sum_c softmax(s)_c * v_c,  or 0 when R_j is empty.
 * out is double [n_rows][n_kv*q_per_kv][head_dim].
 * n_threads > 0 sets the OpenMP team size (0 = library default).
 */
int oracle_attention(int n_q, int n_kv, int q_per_kv, int head_dim, int page_size,
                     int n_pages, int n_ctx, int sel_cap, const float* q,
                     const int8_t* k_pool, const int8_t* v_pool,
                     const float* k_scale, const float* v_scale,
                     const int32_t* page_table, const int32_t* sel,
                     const int32_t* sel_len, const int32_t* rows, int n_rows,
                     float softmax_scale, double* out, int n_threads) {
  if (n_q < 0 || n_kv < 1 || q_per_kv < 1 || head_dim < 1 || page_size < 1 ||
      n_pages < 1 || n_ctx < 1 || sel_cap < 1)
    return ORACLE_EINVAL;
  if (rows == NULL) n_rows = n_q;
  const int n_qh = n_kv * q_per_kv;
  const double scale = (double)softmax_scale;
  int err = ORACLE_OK;
#ifdef _OPENMP
  const int team = n_threads > 0 ? n_threads : omp_get_max_threads();
#else
  (void)n_threads;
#endif
  #pragma omp parallel num_threads(team)
  {
    int32_t* cells = (int32_t*)malloc(sizeof(int32_t) * (size_t)sel_cap);
    int32_t* phys = (int32_t*)malloc(sizeof(int32_t) * (size_t)sel_cap);
    double* s = (double*)malloc(sizeof(double) * (size_t)sel_cap);
    double* kv = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!cells || !phys || !s || !kv) {
      #pragma omp critical
      err = ORACLE_ENOMEM;
    }
    #pragma omp for schedule(dynamic, 8)
    for (int r = 0; r < n_rows; ++r) {
      if (!cells || !phys || !s || !kv) continue;
      const int j = rows ? rows[r] : r;
      double* o_row = out + (size_t)r * n_qh * head_dim;
      int len = (j >= 0 && j < n_q) ? sel_len[j] : -1;
      int n = -1;
      if (len >= 0 && len <= sel_cap)
        n = row_as_set(sel + (size_t)j * sel_cap, len, n_ctx, cells);
      if (n < 0) {
        #pragma omp critical
        err = ORACLE_EINVAL;
        continue;
      }
      /* keep the cells whose page is resident; remember where each one lives */
      int m = 0;
      for (int e = 0; e < n; ++e) {
        const int32_t pp = page_table[cells[e] / page_size];
        if (pp < 0) continue;
        if (pp >= n_pages) {
          #pragma omp critical
          err = ORACLE_EINVAL;
          continue;
        }
        cells[m] = cells[e];
        phys[m] = pp;
        ++m;
      }
      for (int h = 0; h < n_qh; ++h) {
        const int kvh = h / q_per_kv;
        const float* qv = q + ((size_t)j * n_qh + h) * head_dim;
        double* o = o_row + (size_t)h * head_dim;
        for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
        if (m == 0) continue;
        /* scores */
        double smax = -INFINITY;
        for (int e = 0; e < m; ++e) {
          const int t = cells[e] % page_size;
          const size_t base = (((size_t)phys[e] * n_kv + kvh) * page_size + t);
          const double ks = (double)k_scale[base];
          const int8_t* krow = k_pool + base * head_dim;
          double dot = 0.0;
          for (int d = 0; d < head_dim; ++d) dot += (double)qv[d] * ((double)krow[d] * ks);
          s[e] = scale * dot;
          if (s[e] > smax) smax = s[e];
        }
        /* softmax weights */
        double z = 0.0;
        for (int e = 0; e < m; ++e) {
          s[e] = exp(s[e] - smax);
          z += s[e];
        }
        /* weighted sum of the dequantised values */
        for (int e = 0; e < m; ++e) {
          const int t = cells[e] % page_size;
          const size_t base = (((size_t)phys[e] * n_kv + kvh) * page_size + t);
          const double vs = (double)v_scale[base];
          const int8_t* vrow = v_pool + base * head_dim;
          const double w = s[e] / z;
          for (int d = 0; d < head_dim; ++d) kv[d] = (double)vrow[d] * vs;
          for (int d = 0; d < head_dim; ++d) o[d] += w * kv[d];
        }
      }
    }
    free(cells);
    free(phys);
    free(s);
    free(kv);
  }
  return err;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
