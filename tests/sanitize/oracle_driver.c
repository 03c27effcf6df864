/*
 * oracle_driver.c -- runs every entry point of the CPU oracle (oracle/gdn_oracle.c)
 * on small inputs, valid and invalid, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer sees each code path once: out-of-bounds accesses,
 * leaks, overflow and misaligned accesses abort the run.  Test infrastructure:
 * tests/test_sanitizers.py compiles and runs it; nothing else uses it.
 * Exit status 0: every call returned the status expected of it.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_f64(uint16_t h);
int oracle_run(int Hk, int Hv, int dk, int dv, int W, double* S, double* tail, const void* w, int w_bf16, int T,
               const void* x, int x_bf16, const int32_t* rows, const float* a, const float* b, double* o, int h_lo,
               int h_hi);
int oracle_recur(int Hk, int Hv, int dk, int dv, double* S, const double* y, const double* a, const double* b,
                 double* o);
int oracle_run_kda(int Hk, int Hv, int dk, int dv, int W, double* S, double* tail, const void* w, int w_bf16, int T,
                   const void* x, int x_bf16, const float* a, const float* b, double* o);
int oracle_recur_kda(int Hk, int Hv, int dk, int dv, double* S, const double* y, const double* a, const double* b,
                     double* o);
int oracle_conv(int C, int W, double* tail, const void* w, int w_bf16, int T, const void* x, int x_bf16, double* y);
int oracle_tree_tables(int n, const int32_t* parent, int max_depth, int32_t* depth, int32_t* order);
int oracle_tree_verify(int Hk, int Hv, int dk, int dv, int W, const double* S_c, const double* tail_c, const void* w,
                       int w_bf16, int n, const int32_t* parent, int max_depth, const void* x, int x_bf16,
                       const float* a, const float* b, double* o, int h_lo, int h_hi);
int oracle_commit_path(int Hk, int Hv, int dk, int dv, int W, double* S, double* tail, const void* w, int w_bf16,
                       int n, const int32_t* parent, int max_depth, const void* x, int x_bf16, const float* a,
                       const float* b, int L, const int32_t* path, double* o, int h_lo, int h_hi);

static uint64_t rng = 88172645463325252ull;
static double urand(void)  /* xorshift64, uniform in [-1, 1) */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}
static double* drand_arr(size_t n)
{
    double* p = xmalloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i)
        p[i] = urand();
    return p;
}
static float* frand_arr(size_t n)
{
    float* p = xmalloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i)
        p[i] = (float)(2.0 * urand());
    return p;
}
static uint16_t* brand_arr(size_t n)  /* bf16 bit patterns of values in [-1, 1) */
{
    uint16_t* p = xmalloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) {
        float f = (float)urand();
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        p[i] = (uint16_t)(u >> 16);
    }
    return p;
}

static int failures = 0;
static void expect(const char* what, int got, int want)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

static void run_shape(int Hk, int Hv, int dk, int dv, int bf16)
{
    const int W = 4, C = 2 * Hk * dk + Hv * dv, T = 9, n = 12;
    const size_t s_n = (size_t)Hv * dv * dk;
    double* S = drand_arr(s_n);
    double* tail = drand_arr((size_t)C * W);
    void* w = bf16 ? (void*)brand_arr((size_t)C * W) : (void*)frand_arr((size_t)C * W);
    void* x = bf16 ? (void*)brand_arr((size_t)T * C) : (void*)frand_arr((size_t)T * C);
    float* a = frand_arr((size_t)T * Hv);
    float* b = frand_arr((size_t)T * Hv);
    float* ak = frand_arr((size_t)T * Hv * dk);
    double* o = xmalloc((size_t)T * Hv * dv * sizeof(double));
    int32_t rows[9] = {8, 0, 3, 3, 7, 1, 2, 6, 5};

    expect("run", oracle_run(Hk, Hv, dk, dv, W, S, tail, w, bf16, T, x, bf16, NULL, a, b, o, 0, Hv), 0);
    expect("run rows", oracle_run(Hk, Hv, dk, dv, W, S, tail, w, bf16, T, x, bf16, rows, a, b, NULL, 0, Hv), 0);
    expect("run head range", oracle_run(Hk, Hv, dk, dv, W, S, tail, w, bf16, T, x, bf16, NULL, a, b, o, 1, Hv), 0);
    expect("run T=0", oracle_run(Hk, Hv, dk, dv, W, S, tail, w, bf16, 0, x, bf16, NULL, a, b, o, 0, Hv), 0);
    expect("run bad range", oracle_run(Hk, Hv, dk, dv, W, S, tail, w, bf16, T, x, bf16, NULL, a, b, o, 0, Hv + 1), 1);
    expect("run bad group", oracle_run(2, 3, dk, dv, W, S, tail, w, bf16, T, x, bf16, NULL, a, b, o, 0, 1), 1);
    expect("run_kda", oracle_run_kda(Hk, Hv, dk, dv, W, S, tail, w, bf16, T, x, bf16, ak, b, o), 0);
    expect("run_kda no o", oracle_run_kda(Hk, Hv, dk, dv, W, S, tail, w, bf16, T, x, bf16, ak, b, NULL), 0);
    expect("run_kda bad dims", oracle_run_kda(0, Hv, dk, dv, W, S, tail, w, bf16, T, x, bf16, ak, b, o), 1);

    double* y = drand_arr((size_t)C);
    double* ad = drand_arr((size_t)Hv * dk);
    double* bd = drand_arr((size_t)Hv);
    expect("recur", oracle_recur(Hk, Hv, dk, dv, S, y, ad, bd, o), 0);
    expect("recur_kda", oracle_recur_kda(Hk, Hv, dk, dv, S, y, ad, bd, o), 0);
    double* yc = xmalloc((size_t)T * C * sizeof(double));
    expect("conv", oracle_conv(C, W, tail, w, bf16, T, x, bf16, yc), 0);
    expect("conv bad", oracle_conv(C, 0, tail, w, bf16, T, x, bf16, yc), 1);

    /* a tree of n nodes: node i hangs under i / 2 (depth <= 4); x/a/b hold one row per node */
    int32_t parent[12], depth[12], order[12];
    parent[0] = -1;
    for (int i = 1; i < n; ++i)
        parent[i] = i / 2;
    void* xt = bf16 ? (void*)brand_arr((size_t)n * C) : (void*)frand_arr((size_t)n * C);
    float* at = frand_arr((size_t)n * Hv);
    float* bt = frand_arr((size_t)n * Hv);
    double* ot = xmalloc((size_t)n * Hv * dv * sizeof(double));
    expect("tables", oracle_tree_tables(n, parent, 8, depth, order), 0);
    expect("tables depth", oracle_tree_tables(n, parent, 3, depth, order), 2);
    expect("verify", oracle_tree_verify(Hk, Hv, dk, dv, W, S, tail, w, bf16, n, parent, 8, xt, bf16, at, bt, ot, 0,
                                        Hv), 0);
    int32_t path[4] = {0, 1, 3, 7};
    expect("commit", oracle_commit_path(Hk, Hv, dk, dv, W, S, tail, w, bf16, n, parent, 8, xt, bf16, at, bt, 4, path,
                                        o, 0, Hv), 0);
    int32_t bad_path[4] = {0, 2, 3, 7};
    expect("commit non-path", oracle_commit_path(Hk, Hv, dk, dv, W, S, tail, w, bf16, n, parent, 8, xt, bf16, at, bt, 4,
                                                 bad_path, o, 0, Hv), 2);
    int32_t out_of_range[2] = {0, 40};
    expect("commit out of range", oracle_commit_path(Hk, Hv, dk, dv, W, S, tail, w, bf16, n, parent, 8, xt, bf16, at,
                                                     bt, 2, out_of_range, o, 0, Hv), 2);
    parent[5] = 9;  /* a parent after its child */
    expect("tables malformed", oracle_tree_tables(n, parent, 8, depth, order), 2);
    expect("verify malformed", oracle_tree_verify(Hk, Hv, dk, dv, W, S, tail, w, bf16, n, parent, 8, xt, bf16, at, bt,
                                                  ot, 0, Hv), 2);
    parent[0] = 0;  /* a root with a parent */
    expect("tables bad root", oracle_tree_tables(n, parent, 8, depth, order), 2);

    for (size_t i = 0; i < s_n; ++i)
        if (!isfinite(S[i])) {
            fprintf(stderr, "state not finite\n");
            ++failures;
            break;
        }
    free(S); free(tail); free(w); free(x); free(a); free(b); free(ak); free(o); free(y); free(ad); free(bd);
    free(yc); free(xt); free(at); free(bt); free(ot);
}

int main(void)
{
    for (uint32_t h = 0; h < 65536; h += 257)
        (void)oracle_bf16_to_f64((uint16_t)h);
    run_shape(1, 1, 4, 4, 0);
    run_shape(2, 6, 8, 12, 1);   /* grouped 3:1, dk != dv */
    run_shape(4, 4, 32, 32, 0);  /* the tiny layer */
    if (failures) {
        fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    printf("oracle driver: every call as expected\n");
    return 0;
}
