/*
 * Oracle: plain, slow, CPU-only exact tensor-network contraction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this; it is
 * used by the tests, the smoke check and the CPU-baseline leg of the bench.
 * It shares no code, header or table with the GPU library.
 *
 * What it computes (source page "Parallelizing Large-Scale Tensor Network
 * Contraction on Multiple GPUs", section 1.1, the pairwise contraction step):
 * each step of the tree forms C = sum over the modes K shared by A and B of
 * A * B, where the retained modes of A (M) and of B (N) survive into C.  The
 * whole tree therefore evaluates the network's full sum
 *     out[o] = sum over all closed-mode assignments of prod_leaves T_leaf,
 * only in a particular bracketing.  This file evaluates the steps one by one
 * in the most direct way:
 *   - leaves are widened to complex128 (interleaved re, im doubles);
 *   - C is stored in its natural order [M in A's order | N in B's order];
 *   - each entry of C is a sequential sum over every assignment of K,
 *     enumerated with a mixed-radix counter;
 *   - output entries are distributed over OpenMP threads;
 *   - the root is finally permuted into the requested output order.
 * Optional "fixed" modes pin a closed mode to one value in every leaf that
 * carries it, which evaluates one term of the sum over that mode (a slice).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NETWORK 2
#define ORC_ERR_TREE 3
#define ORC_ERR_NOMEM 5

typedef struct {
  int rank;
  int32_t *modes;   /* row-major order, first = slowest */
  int64_t *dims;
  int64_t size;     /* number of complex entries */
  double *data;     /* 2*size doubles */
} otensor;

static void ot_free(otensor *t) {
  free(t->modes); free(t->dims); free(t->data);
  memset(t, 0, sizeof(*t));
}

static int ot_alloc(otensor *t, int rank) {
  t->rank = rank;
  t->modes = (int32_t *)malloc(sizeof(int32_t) * (rank > 0 ? rank : 1));
  t->dims = (int64_t *)malloc(sizeof(int64_t) * (rank > 0 ? rank : 1));
  t->data = NULL;
  return (t->modes && t->dims) ? ORC_OK : ORC_ERR_NOMEM;
}

/* Row-major strides of a tensor (in complex entries). */
static void strides_of(const otensor *t, int64_t *st) {
  int64_t s = 1;
  for (int p = t->rank - 1; p >= 0; --p) { st[p] = s; s *= t->dims[p]; }
}

static int find_mode(const otensor *t, int32_t x) {
  for (int p = 0; p < t->rank; ++p) if (t->modes[p] == x) return p;
  return -1;
}

/* One pairwise step in natural layout: C[M | N] = sum_K A[M, K] B[N, K]. */
static int contract_pair(const otensor *A, const otensor *B, otensor *C, int nthreads) {
  int ra = A->rank, rb = B->rank;
  int64_t *sa = (int64_t *)malloc(sizeof(int64_t) * (ra + 1));
  int64_t *sb = (int64_t *)malloc(sizeof(int64_t) * (rb + 1));
  strides_of(A, sa); strides_of(B, sb);

  /* classify modes */
  int nm = 0, nn = 0, nk = 0;
  int *mpos = (int *)malloc(sizeof(int) * (ra + 1));   /* positions in A of M modes */
  int *npos = (int *)malloc(sizeof(int) * (rb + 1));   /* positions in B of N modes */
  int *kpa = (int *)malloc(sizeof(int) * (ra + 1));    /* K positions in A */
  int *kpb = (int *)malloc(sizeof(int) * (ra + 1));    /* same K mode, position in B */
  for (int p = 0; p < ra; ++p) {
    int q = find_mode(B, A->modes[p]);
    if (q < 0) mpos[nm++] = p; else { kpa[nk] = p; kpb[nk] = q; nk++; }
  }
  for (int q = 0; q < rb; ++q)
    if (find_mode(A, B->modes[q]) < 0) npos[nn++] = q;

  int rc = ot_alloc(C, nm + nn);
  if (rc) goto done;
  int64_t csize = 1;
  for (int i = 0; i < nm; ++i) { C->modes[i] = A->modes[mpos[i]]; C->dims[i] = A->dims[mpos[i]]; csize *= C->dims[i]; }
  for (int j = 0; j < nn; ++j) { C->modes[nm + j] = B->modes[npos[j]]; C->dims[nm + j] = B->dims[npos[j]]; csize *= C->dims[nm + j]; }
  C->size = csize;
  C->data = (double *)malloc(sizeof(double) * 2 * (size_t)csize);
  if (!C->data) { rc = ORC_ERR_NOMEM; goto done; }

  int64_t ksize = 1;
  int64_t *kdim = (int64_t *)malloc(sizeof(int64_t) * (nk + 1));
  for (int t = 0; t < nk; ++t) { kdim[t] = A->dims[kpa[t]]; ksize *= kdim[t]; }

#pragma omp parallel num_threads(nthreads)
  {
    int64_t *dig = (int64_t *)malloc(sizeof(int64_t) * (nm + nn + 1));
    int64_t *kd = (int64_t *)malloc(sizeof(int64_t) * (nk + 1));
#pragma omp for schedule(dynamic, 64)
    for (int64_t c = 0; c < csize; ++c) {
      /* digits of c in C's natural order */
      int64_t r = c;
      for (int p = nm + nn - 1; p >= 0; --p) { dig[p] = r % C->dims[p]; r /= C->dims[p]; }
      int64_t oa = 0, ob = 0;
      for (int i = 0; i < nm; ++i) oa += dig[i] * sa[mpos[i]];
      for (int j = 0; j < nn; ++j) ob += dig[nm + j] * sb[npos[j]];
      for (int t = 0; t < nk; ++t) kd[t] = 0;
      double re = 0.0, im = 0.0;
      int64_t ia = oa, ib = ob;   /* offsets of the current K assignment in A and B */
      for (int64_t l = 0; l < ksize; ++l) {
        double ar = A->data[2 * ia], ai = A->data[2 * ia + 1];
        double br = B->data[2 * ib], bi = B->data[2 * ib + 1];
        re += ar * br - ai * bi;
        im += ar * bi + ai * br;
        /* advance the mixed-radix counter over K (last digit fastest),
           moving both offsets by the stride of the digit that changes */
        for (int t = nk - 1; t >= 0; --t) {
          if (++kd[t] < kdim[t]) { ia += sa[kpa[t]]; ib += sb[kpb[t]]; break; }
          ia -= (kdim[t] - 1) * sa[kpa[t]];
          ib -= (kdim[t] - 1) * sb[kpb[t]];
          kd[t] = 0;
        }
      }
      C->data[2 * c] = re;
      C->data[2 * c + 1] = im;
    }
    free(dig); free(kd);
  }
  free(kdim);
done:
  free(sa); free(sb); free(mpos); free(npos); free(kpa); free(kpb);
  return rc;
}

/* Permute T into the mode order `order` (same set of modes). */
static int permute_to(const otensor *T, const int32_t *order, int rank, double *out, int nthreads) {
  int64_t *st = (int64_t *)malloc(sizeof(int64_t) * (T->rank + 1));
  int64_t *srcst = (int64_t *)malloc(sizeof(int64_t) * (rank + 1));
  int64_t *dims = (int64_t *)malloc(sizeof(int64_t) * (rank + 1));
  strides_of(T, st);
  for (int p = 0; p < rank; ++p) {
    int q = find_mode(T, order[p]);
    if (q < 0) { free(st); free(srcst); free(dims); return ORC_ERR_NETWORK; }
    srcst[p] = st[q]; dims[p] = T->dims[q];
  }
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t o = 0; o < T->size; ++o) {
    int64_t r = o, src = 0;
    for (int p = rank - 1; p >= 0; --p) { src += (r % dims[p]) * srcst[p]; r /= dims[p]; }
    out[2 * o] = T->data[2 * src];
    out[2 * o + 1] = T->data[2 * src + 1];
  }
  free(st); free(srcst); free(dims);
  return ORC_OK;
}

/*
 * Contract a whole network along a tree.
 *   extents[num_modes]            mode extents
 *   leaf_rank[L], leaf_modes[...]  declared mode order of each leaf
 *   leaf_data[L]                   row-major buffers: complex64 (interleaved float re, im),
 *                                  or complex128 (interleaved double) when leaf_c128 != 0
 *   lhs[S], rhs[S]                 SSA operand ids; step s creates L + s
 *   out_modes[out_rank]            output order
 *   fixed_modes/values[num_fixed]  closed modes pinned to one value
 *   out                            complex128 result (2 * prod(out extents) doubles)
 */
int oracle_contract(int32_t num_modes, const int64_t *extents,
                    int32_t num_leaves, const int32_t *leaf_rank, const int32_t *leaf_modes,
                    const void *const *leaf_data, int32_t leaf_c128,
                    int32_t num_steps, const int32_t *lhs, const int32_t *rhs,
                    int32_t out_rank, const int32_t *out_modes,
                    int32_t num_fixed, const int32_t *fixed_modes, const int64_t *fixed_values,
                    double *out, int32_t nthreads) {
  if (num_leaves < 1 || num_steps != num_leaves - 1) return ORC_ERR_TREE;
  if (nthreads < 1) nthreads = 1;
  int total = num_leaves + num_steps;
  otensor *T = (otensor *)calloc((size_t)total, sizeof(otensor));
  if (!T) return ORC_ERR_NOMEM;
  int rc = ORC_OK;

  /* leaves, with fixed modes removed */
  int64_t off = 0;
  for (int l = 0; l < num_leaves && rc == ORC_OK; ++l) {
    int r = leaf_rank[l];
    const int32_t *lm = leaf_modes + off;
    off += r;
    int64_t *full_st = (int64_t *)malloc(sizeof(int64_t) * (r + 1));
    int64_t s = 1;
    for (int p = r - 1; p >= 0; --p) {
      if (lm[p] < 0 || lm[p] >= num_modes) { rc = ORC_ERR_NETWORK; break; }
      full_st[p] = s; s *= extents[lm[p]];
    }
    if (rc) { free(full_st); break; }
    int64_t base = 0;
    int keep = 0;
    for (int p = 0; p < r; ++p) {
      int fixed = -1;
      for (int f = 0; f < num_fixed; ++f) if (fixed_modes[f] == lm[p]) fixed = f;
      if (fixed >= 0) base += fixed_values[fixed] * full_st[p]; else keep++;
    }
    rc = ot_alloc(&T[l], keep);
    if (rc) { free(full_st); break; }
    int64_t *kst = (int64_t *)malloc(sizeof(int64_t) * (keep + 1));
    int q = 0;
    int64_t size = 1;
    for (int p = 0; p < r; ++p) {
      int fixed = 0;
      for (int f = 0; f < num_fixed; ++f) if (fixed_modes[f] == lm[p]) fixed = 1;
      if (fixed) continue;
      T[l].modes[q] = lm[p]; T[l].dims[q] = extents[lm[p]]; kst[q] = full_st[p];
      size *= extents[lm[p]]; q++;
    }
    T[l].size = size;
    T[l].data = (double *)malloc(sizeof(double) * 2 * (size_t)size);
    for (int64_t e = 0; e < size; ++e) {
      int64_t rr = e, src = base;
      for (int p = keep - 1; p >= 0; --p) { src += (rr % T[l].dims[p]) * kst[p]; rr /= T[l].dims[p]; }
      if (leaf_c128) {
        const double *d = (const double *)leaf_data[l];
        T[l].data[2 * e] = d[2 * src];
        T[l].data[2 * e + 1] = d[2 * src + 1];
      } else {
        const float *f = (const float *)leaf_data[l];
        T[l].data[2 * e] = (double)f[2 * src];
        T[l].data[2 * e + 1] = (double)f[2 * src + 1];
      }
    }
    free(kst); free(full_st);
  }

  /* steps in list order */
  for (int s = 0; s < num_steps && rc == ORC_OK; ++s) {
    int a = lhs[s], b = rhs[s];
    if (a < 0 || b < 0 || a >= num_leaves + s || b >= num_leaves + s || a == b ||
        T[a].data == NULL || T[b].data == NULL) { rc = ORC_ERR_TREE; break; }
    rc = contract_pair(&T[a], &T[b], &T[num_leaves + s], nthreads);
    ot_free(&T[a]); ot_free(&T[b]);
  }

  if (rc == ORC_OK) {
    otensor *R = &T[total - 1];
    if (R->rank != out_rank) rc = ORC_ERR_NETWORK;
    else rc = permute_to(R, out_modes, out_rank, out, nthreads);
  }
  for (int i = 0; i < total; ++i) ot_free(&T[i]);
  free(T);
  return rc;
}

/*
 * Sampled entries of one pairwise contraction: out[s] = sum_l a[s*k + l] * b[s*k + l]
 * for s < count, in complex128.  The caller gathers, for each sampled output
 * entry, the k entries of A and of B that meet in it (same K assignment at
 * the same position l); this routine is the plain sum of their products.
 */
void oracle_dot_rows(int64_t count, int64_t k, const float *a, const float *b, double *out, int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t s = 0; s < count; ++s) {
    double re = 0.0, im = 0.0;
    for (int64_t l = 0; l < k; ++l) {
      double ar = a[2 * (s * k + l)], ai = a[2 * (s * k + l) + 1];
      double br = b[2 * (s * k + l)], bi = b[2 * (s * k + l) + 1];
      re += ar * br - ai * bi;
      im += ar * bi + ai * br;
    }
    out[2 * s] = re;
    out[2 * s + 1] = im;
  }
}

/*
 * A block of one pairwise contraction: out[i*nj + j] = sum_l a[i*k + l] * b[j*k + l]
 * for the ni gathered rows of A and nj gathered rows of B (both complex64,
 * K innermost), in complex128.  This is C = sum_K A[M, K] B[N, K] restricted
 * to a sub-grid of output entries.
 */
void oracle_pair_block(int64_t ni, int64_t nj, int64_t k, const float *a, const float *b, double *out,
                       int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) collapse(2)
  for (int64_t i = 0; i < ni; ++i) {
    for (int64_t j = 0; j < nj; ++j) {
      double re = 0.0, im = 0.0;
      for (int64_t l = 0; l < k; ++l) {
        double ar = a[2 * (i * k + l)], ai = a[2 * (i * k + l) + 1];
        double br = b[2 * (j * k + l)], bi = b[2 * (j * k + l) + 1];
        re += ar * br - ai * bi;
        im += ar * bi + ai * br;
      }
      out[2 * (i * nj + j)] = re;
      out[2 * (i * nj + j) + 1] = im;
    }
  }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
