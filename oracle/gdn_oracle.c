/*
 * gdn_oracle.c -- the CPU oracle of the Gated DeltaNet recurrent mixer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
 * baseline load this file's library.  The HIP library never includes, links
 * or calls it, and it shares no code with the HIP library.
 *
 * What it is: the plain sequential definition, token by token, in double
 * precision, with every sum taken left to right from index 0.  It follows the
 * serving-engine pages' statement of the problem:
 *   - "Architecture", section 8.1 and its table: each recurrent layer keeps a
 *     fixed-size fp32 state per head (48 heads of 128 by 128) and a 4-wide
 *     convolution tail, and the engine must be able to undo it exactly,
 *     branch it over a tree of guesses and restore it;
 *   - "Serving a research architecture on CPU" (the constant-state section):
 *     each head's [d, d] state is updated in place by a rank-1 outer product
 *     every token, and short convolutions carry rings of recent activations;
 *     16-bit stored values are widened exactly before fp32 (here fp64)
 *     arithmetic; the scalar path is the definition the fast paths answer to.
 * The pages never print the recurrence itself.  The readings used (decay
 * before the delta correction, output from the updated state, q/k L2 norm
 * with eps = 1e-6, alpha = exp(-softplus(a)), beta = sigmoid(b), o scaled by
 * 1/sqrt(dk), value head h served by q/k head h / (Hv/Hk)) are the plainest
 * form of the "gated delta rule" with these gates and this output.
 *
 * Per token, for one sequence:
 *   conv   y[c]   = SiLU( sum_j w[c][j] * win[c][j] ),  win = last W raw inputs
 *   split  q~ = y[g*dk ..], k~ = y[Hk*dk + g*dk ..], v = y[2*Hk*dk + h*dv ..]
 *   norm   q^ = q~ / sqrt(sum q~^2 + eps), same for k^
 *   gates  alpha = exp(-softplus(a)), beta = 1 / (1 + exp(-b))
 *   state  S <- alpha*S;  p = S k^;  S <- S + beta*(v - p) k^T;  o = S q^ / sqrt(dk)
 * with S stored as rows over the value index, each row contiguous over keys.
 *
 * Parity pins (tests/test_oracle_pins.py): exhaustive bf16 widening; conv
 * against a direct full-sequence convolution; a hand-derived 2x2 example;
 * a brute-force unrolled product of transition matrices; closed forms at
 * beta = 0, at alpha = beta = 1 and at T = 1; group mapping; tree and path
 * invariants; the chunked (WY) form derived independently in NumPy.
 * The per-channel-decay variant (oracle_run_kda) is pinned in
 * tests/test_oracle_kda.py: scalar gates equal oracle_run bit for bit, beta = 0
 * leaves S0 diag(prod alpha), a worked one-hot-key step, and the brute-force
 * product of its transition matrices.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EPS 1e-6

enum { ORACLE_OK = 0, ORACLE_ERR_ARG = 1, ORACLE_ERR_TREE = 2 };

/* ------------------------------------------------------------ storage widening */

/* bf16 is the top half of an IEEE binary32; widening is exact ("Serving a
 * research architecture on CPU", exactness paragraphs: 16-bit stored values
 * are converted exactly before arithmetic). */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double load_act(const void* p, int is_bf16, size_t i)
{
    if (is_bf16)
        return oracle_bf16_to_f64(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

/* ------------------------------------------------------------ scalar pieces */

static double silu(double z) { return z / (1.0 + exp(-z)); }
static double softplus(double a) { return fmax(a, 0.0) + log1p(exp(-fabs(a))); }
static double sigmoid(double b) { return 1.0 / (1.0 + exp(-b)); }

/* ------------------------------------------------------------ layer geometry */

typedef struct {
    int Hk, Hv, dk, dv, W, C, G;
} geom;

static int make_geom(geom* g, int Hk, int Hv, int dk, int dv, int W)
{
    if (Hk < 1 || Hv < 1 || dk < 1 || dv < 1 || W < 1 || Hv % Hk != 0)
        return ORACLE_ERR_ARG;
    g->Hk = Hk; g->Hv = Hv; g->dk = dk; g->dv = dv; g->W = W;
    g->C = 2 * Hk * dk + Hv * dv;
    g->G = Hv / Hk;
    return ORACLE_OK;
}

/* Channels the v heads [h_lo, h_hi) read: the q and k channels of their q/k
 * heads and their own v channels. */
static void mark_needed(const geom* g, int h_lo, int h_hi, unsigned char* need)
{
    memset(need, 0, (size_t)g->C);
    for (int h = h_lo; h < h_hi; ++h) {
        int kh = h / g->G;
        for (int c = 0; c < g->dk; ++c) {
            need[kh * g->dk + c] = 1;
            need[g->Hk * g->dk + kh * g->dk + c] = 1;
        }
        for (int i = 0; i < g->dv; ++i)
            need[2 * g->Hk * g->dk + h * g->dv + i] = 1;
    }
}

/* One token of the causal depthwise conv.  tail[c][0..W-1] holds the last W
 * raw inputs, oldest first; it shifts by one and takes x[c] as the newest,
 * then y[c] = SiLU(sum_j w[c][j] * tail[c][j]) for the channels marked.
 * ("Architecture" section 8.1 table: a 4-wide convolution tail per layer;
 * CPU page, constant-state paragraph: short convolutions keep rings of
 * recent inputs.) */
static void conv_token(const geom* g, double* tail, const void* w, int w_bf16,
                       const void* x, int x_bf16, size_t x_off,
                       const unsigned char* need, double* y)
{
    for (int c = 0; c < g->C; ++c) {
        double* t = tail + (size_t)c * g->W;
        for (int j = 0; j + 1 < g->W; ++j)
            t[j] = t[j + 1];
        t[g->W - 1] = load_act(x, x_bf16, x_off + (size_t)c);
        if (!need[c])
            continue;
        double acc = 0.0;
        for (int j = 0; j < g->W; ++j)
            acc = acc + load_act(w, w_bf16, (size_t)c * g->W + j) * t[j];
        y[c] = silu(acc);
    }
}

/* One token of the recurrence for v heads [h_lo, h_hi), given the conv output
 * y.  S is [Hv][dv][dk]; o (nullable) is [Hv][dv].  ("Architecture" section
 * 8.1: a fixed-size fp32 state per head, advanced per token; CPU page,
 * constant-state paragraph: a rank-1 outer-product update of each head's
 * square state, in place.) */
static void recur_token(const geom* g, double* S, const double* y, const double* a, const double* b,
                        double* o, int h_lo, int h_hi, double* qh, double* kh)
{
    const double scale = 1.0 / sqrt((double)g->dk);
    for (int h = h_lo; h < h_hi; ++h) {
        const int grp = h / g->G;
        const double* q = y + (size_t)grp * g->dk;
        const double* k = y + (size_t)g->Hk * g->dk + (size_t)grp * g->dk;
        const double* v = y + (size_t)2 * g->Hk * g->dk + (size_t)h * g->dv;

        double nq = 0.0, nk = 0.0;
        for (int c = 0; c < g->dk; ++c) {
            nq = nq + q[c] * q[c];
            nk = nk + k[c] * k[c];
        }
        const double rq = 1.0 / sqrt(nq + ORACLE_EPS);
        const double rk = 1.0 / sqrt(nk + ORACLE_EPS);
        for (int c = 0; c < g->dk; ++c) {
            qh[c] = q[c] * rq;
            kh[c] = k[c] * rk;
        }

        const double alpha = exp(-softplus(a[h]));
        const double beta = sigmoid(b[h]);

        for (int i = 0; i < g->dv; ++i) {
            double* row = S + ((size_t)h * g->dv + i) * g->dk;
            for (int c = 0; c < g->dk; ++c)
                row[c] = alpha * row[c];
            double p = 0.0;
            for (int c = 0; c < g->dk; ++c)
                p = p + row[c] * kh[c];
            const double u = beta * (v[i] - p);
            for (int c = 0; c < g->dk; ++c)
                row[c] = row[c] + u * kh[c];
            if (o) {
                double r = 0.0;
                for (int c = 0; c < g->dk; ++c)
                    r = r + row[c] * qh[c];
                o[(size_t)h * g->dv + i] = scale * r;
            }
        }
    }
}

/* ------------------------------------------------------------ exported calls */

/*
 * oracle_run: T tokens of one sequence from (S, tail), in place: the
 * token-by-token definition (CPU page, exactness paragraphs: the scalar path
 * is what the fast paths answer to).
 *   S     double [Hv][dv][dk]          in/out
 *   tail  double [C][W]                in/out (raw inputs, oldest first)
 *   w     act   [C][W]   (bf16 bits if w_bf16 else float)
 *   x     act   token t at x + rows[t] * C (rows == NULL: row t)
 *   a, b  float token t at a + rows[t] * Hv
 *   o     double [T][Hv][dv] (nullable)
 *   v heads [h_lo, h_hi) are advanced; other heads of S are left as they are.
 *   The tail always advances on every channel.
 */
int oracle_run(int Hk, int Hv, int dk, int dv, int W,
               double* S, double* tail, const void* w, int w_bf16,
               int T, const void* x, int x_bf16, const int32_t* rows,
               const float* a, const float* b, double* o, int h_lo, int h_hi)
{
    geom g;
    if (make_geom(&g, Hk, Hv, dk, dv, W) != ORACLE_OK || T < 0 || h_lo < 0 || h_hi > Hv || h_lo > h_hi)
        return ORACLE_ERR_ARG;
    unsigned char* need = malloc((size_t)g.C);
    double* y = calloc((size_t)g.C, sizeof(double));
    double* qh = malloc((size_t)dk * sizeof(double));
    double* kh = malloc((size_t)dk * sizeof(double));
    double* ah = malloc((size_t)Hv * sizeof(double));
    double* bh = malloc((size_t)Hv * sizeof(double));
    if (!need || !y || !qh || !kh || !ah || !bh) {
        free(need); free(y); free(qh); free(kh); free(ah); free(bh);
        return ORACLE_ERR_ARG;
    }
    mark_needed(&g, h_lo, h_hi, need);
    for (int t = 0; t < T; ++t) {
        const size_t r = rows ? (size_t)rows[t] : (size_t)t;
        conv_token(&g, tail, w, w_bf16, x, x_bf16, r * (size_t)g.C, need, y);
        for (int h = 0; h < Hv; ++h) {
            ah[h] = (double)a[r * (size_t)Hv + h];
            bh[h] = (double)b[r * (size_t)Hv + h];
        }
        recur_token(&g, S, y, ah, bh, o ? o + (size_t)t * Hv * dv : NULL, h_lo, h_hi, qh, kh);
    }
    free(need); free(y); free(qh); free(kh); free(ah); free(bh);
    return ORACLE_OK;
}

/*
 * oracle_recur (same passages as recur_token): one token of the recurrence alone, from a given conv output
 * y[C] (already split as q|k|v) and gate inputs a[Hv], b[Hv].  All heads.
 */
int oracle_recur(int Hk, int Hv, int dk, int dv, double* S, const double* y,
                 const double* a, const double* b, double* o)
{
    geom g;
    if (make_geom(&g, Hk, Hv, dk, dv, 1) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    double* qh = malloc((size_t)dk * sizeof(double));
    double* kh = malloc((size_t)dk * sizeof(double));
    double* ah = malloc((size_t)Hv * sizeof(double));
    double* bh = malloc((size_t)Hv * sizeof(double));
    if (!qh || !kh || !ah || !bh) {
        free(qh); free(kh); free(ah); free(bh);
        return ORACLE_ERR_ARG;
    }
    for (int h = 0; h < Hv; ++h) { ah[h] = a[h]; bh[h] = b[h]; }
    recur_token(&g, S, y, ah, bh, o, 0, Hv, qh, kh);
    free(qh); free(kh); free(ah); free(bh);
    return ORACLE_OK;
}

/* ------------------------------------------------------------ per-channel decay */

/*
 * The per-channel-decay delta rule (the model-arch page's module list names a
 * Kimi Delta Attention mixer with a CPU reference and GPU launches, and does
 * not define it).  Reading taken here: the conv, the q/k norm, beta and the
 * output are those of the gated delta rule above; only the forget gate
 * changes, from one scalar per value head to one value per (value head, key
 * channel):
 *   alpha[c] = exp(-softplus(a[h][c]))
 *   S <- S diag(alpha);  p = S k^;  S <- S + beta*(v - p) k^T;  o = S q^ / sqrt(dk)
 * so column c of every row (key channel c) decays by its own alpha[c] before
 * the delta correction.  With all alpha[c] equal this is recur_token's step,
 * operation for operation.
 *   a  double [Hv][dk] (this token's per-channel gate inputs)
 */
static void recur_token_kda(const geom* g, double* S, const double* y, const double* a, const double* b,
                            double* o, double* qh, double* kh, double* al)
{
    const double scale = 1.0 / sqrt((double)g->dk);
    for (int h = 0; h < g->Hv; ++h) {
        const int grp = h / g->G;
        const double* q = y + (size_t)grp * g->dk;
        const double* k = y + (size_t)g->Hk * g->dk + (size_t)grp * g->dk;
        const double* v = y + (size_t)2 * g->Hk * g->dk + (size_t)h * g->dv;

        double nq = 0.0, nk = 0.0;
        for (int c = 0; c < g->dk; ++c) {
            nq = nq + q[c] * q[c];
            nk = nk + k[c] * k[c];
        }
        const double rq = 1.0 / sqrt(nq + ORACLE_EPS);
        const double rk = 1.0 / sqrt(nk + ORACLE_EPS);
        for (int c = 0; c < g->dk; ++c) {
            qh[c] = q[c] * rq;
            kh[c] = k[c] * rk;
            al[c] = exp(-softplus(a[(size_t)h * g->dk + c]));
        }
        const double beta = sigmoid(b[h]);

        for (int i = 0; i < g->dv; ++i) {
            double* row = S + ((size_t)h * g->dv + i) * g->dk;
            for (int c = 0; c < g->dk; ++c)
                row[c] = al[c] * row[c];
            double p = 0.0;
            for (int c = 0; c < g->dk; ++c)
                p = p + row[c] * kh[c];
            const double u = beta * (v[i] - p);
            for (int c = 0; c < g->dk; ++c)
                row[c] = row[c] + u * kh[c];
            if (o) {
                double r = 0.0;
                for (int c = 0; c < g->dk; ++c)
                    r = r + row[c] * qh[c];
                o[(size_t)h * g->dv + i] = scale * r;
            }
        }
    }
}

/*
 * oracle_run_kda (same passages as recur_token_kda and conv_token): T tokens
 * of one sequence with the per-channel forget gate, in place, all heads.
 *   S     double [Hv][dv][dk]   in/out
 *   tail  double [C][W]         in/out
 *   w, x  act as in oracle_run (x token t at row t)
 *   a     float  [T][Hv][dk]    per-channel gate inputs
 *   b     float  [T][Hv]
 *   o     double [T][Hv][dv]    (nullable)
 */
int oracle_run_kda(int Hk, int Hv, int dk, int dv, int W,
                   double* S, double* tail, const void* w, int w_bf16,
                   int T, const void* x, int x_bf16,
                   const float* a, const float* b, double* o)
{
    geom g;
    if (make_geom(&g, Hk, Hv, dk, dv, W) != ORACLE_OK || T < 0)
        return ORACLE_ERR_ARG;
    unsigned char* need = malloc((size_t)g.C);
    double* y = calloc((size_t)g.C, sizeof(double));
    double* qh = malloc((size_t)dk * sizeof(double));
    double* kh = malloc((size_t)dk * sizeof(double));
    double* al = malloc((size_t)dk * sizeof(double));
    double* ah = malloc((size_t)Hv * dk * sizeof(double));
    double* bh = malloc((size_t)Hv * sizeof(double));
    if (!need || !y || !qh || !kh || !al || !ah || !bh) {
        free(need); free(y); free(qh); free(kh); free(al); free(ah); free(bh);
        return ORACLE_ERR_ARG;
    }
    memset(need, 1, (size_t)g.C);
    for (int t = 0; t < T; ++t) {
        conv_token(&g, tail, w, w_bf16, x, x_bf16, (size_t)t * g.C, need, y);
        for (size_t i = 0; i < (size_t)Hv * dk; ++i)
            ah[i] = (double)a[(size_t)t * Hv * dk + i];
        for (int h = 0; h < Hv; ++h)
            bh[h] = (double)b[(size_t)t * Hv + h];
        recur_token_kda(&g, S, y, ah, bh, o ? o + (size_t)t * Hv * dv : NULL, qh, kh, al);
    }
    free(need); free(y); free(qh); free(kh); free(al); free(ah); free(bh);
    return ORACLE_OK;
}

/*
 * oracle_recur_kda (same passages as recur_token_kda): one token of the
 * per-channel-decay recurrence alone, from a given conv output y[C] and gate
 * inputs a[Hv][dk], b[Hv].  All heads.
 */
int oracle_recur_kda(int Hk, int Hv, int dk, int dv, double* S, const double* y,
                     const double* a, const double* b, double* o)
{
    geom g;
    if (make_geom(&g, Hk, Hv, dk, dv, 1) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    double* qh = malloc((size_t)dk * sizeof(double));
    double* kh = malloc((size_t)dk * sizeof(double));
    double* al = malloc((size_t)dk * sizeof(double));
    if (!qh || !kh || !al) {
        free(qh); free(kh); free(al);
        return ORACLE_ERR_ARG;
    }
    recur_token_kda(&g, S, y, a, b, o, qh, kh, al);
    free(qh); free(kh); free(al);
    return ORACLE_OK;
}

/*
 * oracle_conv (same passages as conv_token): T tokens of the conv alone over all C channels.
 *   tail double [C][W] in/out; y double [T][C].
 */
int oracle_conv(int C, int W, double* tail, const void* w, int w_bf16,
                int T, const void* x, int x_bf16, double* y)
{
    if (C < 1 || W < 1 || T < 0)
        return ORACLE_ERR_ARG;
    geom g = {0};
    g.C = C; g.W = W;
    unsigned char* need = malloc((size_t)C);
    if (!need)
        return ORACLE_ERR_ARG;
    memset(need, 1, (size_t)C);
    for (int t = 0; t < T; ++t)
        conv_token(&g, tail, w, w_bf16, x, x_bf16, (size_t)t * C, need, y + (size_t)t * C);
    free(need);
    return ORACLE_OK;
}

/*
 * Draft-tree tables (repository "Architecture" page, decode-loop diagram: a
 * draft tree of up to 32 nodes grown from the last committed token).  A tree
 * of n nodes is a parent array: parent[0] == -1
 * (node 0 is the root, the last committed token) and 0 <= parent[i] < i for
 * i > 0.  depth[root] = 1; depth[i] = depth[parent[i]] + 1 <= max_depth.
 * order[] is the depth-first pre-order that visits children in increasing
 * index.  Returns ORACLE_ERR_TREE if the array is not such a tree.
 */
static int preorder_visit(int n, const int32_t* parent, int node, int32_t* order, int* pos)
{
    order[(*pos)++] = node;
    for (int c = node + 1; c < n; ++c)
        if (parent[c] == node)
            preorder_visit(n, parent, c, order, pos);
    return 0;
}

int oracle_tree_tables(int n, const int32_t* parent, int max_depth, int32_t* depth, int32_t* order)
{
    if (n < 1 || parent[0] != -1)
        return ORACLE_ERR_TREE;
    depth[0] = 1;
    for (int i = 1; i < n; ++i) {
        if (parent[i] < 0 || parent[i] >= i)
            return ORACLE_ERR_TREE;
        depth[i] = depth[parent[i]] + 1;
        if (depth[i] > max_depth)
            return ORACLE_ERR_TREE;
    }
    if (depth[0] > max_depth)
        return ORACLE_ERR_TREE;
    int pos = 0;
    preorder_visit(n, parent, 0, order, &pos);
    return ORACLE_OK;
}

/*
 * oracle_tree_verify (repository "Architecture" page, decode-loop diagram:
 * the whole tree is verified in one pass and the model's token is produced at
 * every node; "Architecture" section 8.1: the state is branched for a tree of
 * guesses): for every node, the output o at that node after running
 * the root-first path to it from copies of the checkpoint (S_c, tail_c).  The
 * checkpoint is not modified.  o is [n][Hv][dv]; heads outside [h_lo, h_hi)
 * are left untouched.  Brute force: each node replays its own path.
 */
int oracle_tree_verify(int Hk, int Hv, int dk, int dv, int W,
                       const double* S_c, const double* tail_c, const void* w, int w_bf16,
                       int n, const int32_t* parent, int max_depth,
                       const void* x, int x_bf16, const float* a, const float* b,
                       double* o, int h_lo, int h_hi)
{
    geom g;
    if (make_geom(&g, Hk, Hv, dk, dv, W) != ORACLE_OK || n < 1)
        return ORACLE_ERR_ARG;
    int32_t* depth = malloc((size_t)n * sizeof(int32_t));
    int32_t* order = malloc((size_t)n * sizeof(int32_t));
    int32_t* path = malloc((size_t)n * sizeof(int32_t));
    const size_t s_elems = (size_t)Hv * dv * dk, t_elems = (size_t)g.C * W;
    double* S = malloc(s_elems * sizeof(double));
    double* tail = malloc(t_elems * sizeof(double));
    double* os = malloc((size_t)n * Hv * dv * sizeof(double));
    int rc = ORACLE_ERR_ARG;
    if (!depth || !order || !path || !S || !tail || !os)
        goto done;
    rc = oracle_tree_tables(n, parent, max_depth, depth, order);
    if (rc != ORACLE_OK)
        goto done;
    for (int node = 0; node < n; ++node) {
        int L = depth[node];
        for (int j = L - 1, m = node; j >= 0; --j, m = parent[m])
            path[j] = m;
        memcpy(S, S_c, s_elems * sizeof(double));
        memcpy(tail, tail_c, t_elems * sizeof(double));
        rc = oracle_run(Hk, Hv, dk, dv, W, S, tail, w, w_bf16, L, x, x_bf16, path, a, b, os, h_lo, h_hi);
        if (rc != ORACLE_OK)
            goto done;
        for (int h = h_lo; h < h_hi; ++h)
            memcpy(o + ((size_t)node * Hv + h) * dv, os + ((size_t)(L - 1) * Hv + h) * dv, (size_t)dv * sizeof(double));
    }
    rc = ORACLE_OK;
done:
    free(depth); free(order); free(path); free(S); free(tail); free(os);
    return rc;
}

/*
 * oracle_commit_path ("Architecture" section 8.1: exact undo and branch of
 * the recurrent state; decode-loop diagram: the accepted tokens are committed):
 * advance (S, tail) in place over an accepted root-first
 * path of the tree (path[0] == 0, parent[path[j]] == path[j-1]).  This is the
 * sequential definition over the path's tokens.  On an invalid path nothing is
 * modified and ORACLE_ERR_TREE is returned.
 */
int oracle_commit_path(int Hk, int Hv, int dk, int dv, int W,
                       double* S, double* tail, const void* w, int w_bf16,
                       int n, const int32_t* parent, int max_depth,
                       const void* x, int x_bf16, const float* a, const float* b,
                       int L, const int32_t* path, double* o, int h_lo, int h_hi)
{
    if (n < 1 || L < 1 || L > n || L > max_depth)
        return ORACLE_ERR_TREE;
    int32_t* depth = malloc((size_t)n * sizeof(int32_t));
    int32_t* order = malloc((size_t)n * sizeof(int32_t));
    if (!depth || !order) {
        free(depth); free(order);
        return ORACLE_ERR_ARG;
    }
    int rc = oracle_tree_tables(n, parent, max_depth, depth, order);
    free(depth); free(order);
    if (rc != ORACLE_OK)
        return rc;
    if (path[0] != 0)
        return ORACLE_ERR_TREE;
    for (int j = 1; j < L; ++j)
        if (path[j] < 0 || path[j] >= n || parent[path[j]] != path[j - 1])
            return ORACLE_ERR_TREE;
    return oracle_run(Hk, Hv, dk, dv, W, S, tail, w, w_bf16, L, x, x_bf16, path, a, b, o, h_lo, h_hi);
}
