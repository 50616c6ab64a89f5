/*
 * SketchSSM decode oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of what the SketchSSM decode path
 * computes, one (sequence, head) tile at a time.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header or constant with the HIP library and never calls it.
 *
 * Sources (the SketchSSM project page, arXiv 2609.33051 and its summaries):
 *  - recurrence S_t = M_t S_{t-1} + B_t, read o_t = S_t^T q_t
 *      (project page, "01 / The idea", full-state equation);
 *  - flush: apply the buffered updates to the full state, then build the
 *    sketch U = S^T Omega from the updated state; the flush step's own output
 *    is computed from the updated state (paper App. B "SketchSSM algorithm";
 *    project page "02 / How to make a sketch", per-window flush panel);
 *  - non-flush read: c_t = C q~_t, o^_t = U c_t, plus the exact contribution
 *    of the buffered updates (project page, per-step non-flush panel;
 *    paper App. D);
 *  - effective query q~_t: the query pulled back through the buffered
 *    transitions, so that the state-read term is S_0^T q~_t (paper Sec. 3.2,
 *    project page error objective; Mamba-2 has decay only, App. C.1);
 *  - ReplaySSM: buffered writes, full-state read each step (paper Sec. 1-2,
 *    App. D);
 *  - dense-fallback heads (rank 0) keep a copy of the state in the sketch
 *    dtype instead of a sketch: the flush writes it, the non-flush read
 *    takes S^T q~ from it (paper App. D: such heads read a bf16 state copy);
 *  - the coefficient map C is either a fixed per-head table (the paper's
 *    fixed-coefficient rule, App. G) or, as the project page's per-window
 *    flush panel has it, the state-dependent map C = (U^T U)^+ U^T S0^T
 *    refreshed at every flush (paper App. A.2.1; App. A.2.2 names the
 *    regularised solve that is written out here);
 *  - the effective query and the buffered term can be evaluated either
 *    serially, one buffered transition at a time, or all at once from a
 *    triangular system over the buffered slots (paper App. C.1, the
 *    WY-style parallel evaluation; the system below is this oracle's
 *    written-out reading of it).
 *
 * Per family (the Mamba-2 write term, the KDA operator order and the gate
 * dtypes are readings taken where the pages leave the step open):
 *   Mamba-2: M = a I, a = exp(-dt * exp(A_h)), B = dt k v^T
 *   GDN:     M = alpha (I - beta k k^T),        B = beta k v^T
 *   KDA:     M = (I - beta k k^T) Diag(g),      B = beta k v^T
 *
 * All arithmetic is fp64.  Values are rounded only where the method stores
 * them: the state S (fp32), the sketch U (fp32 or bf16, via fp32, nearest
 * even) and the output o (activation dtype).  The EXACT store mode keeps
 * fp64 everywhere, for the algebraic pins.
 *
 * A mutation switch plants known mistakes so that a test can show the pins
 * catch them; it is off (0) unless a test sets it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_MAMBA2 = 0, ORC_GDN = 1, ORC_KDA = 2 };
enum { ORC_STORE_EXACT = 0, ORC_STORE_F32 = 1, ORC_STORE_BF16 = 2 };
enum { ORC_OK = 0, ORC_ERR_COUNT = 1 };
enum { ORC_COEF_FIXED = 0, ORC_COEF_STATE = 1 };
enum { ORC_PULLBACK_SERIAL = 0, ORC_PULLBACK_WY = 1, ORC_PULLBACK_PROJ = 2 };

typedef struct {
    int family;
    int dk, dv, W;
    int rmax;          /* row stride of U, Pt, C */
    int state_store;   /* EXACT or F32 */
    int sketch_store;  /* EXACT, F32 or BF16 */
    int out_store;     /* EXACT, F32 or BF16 */
    int coef_mode;     /* ORC_COEF_FIXED: C is an input table;
                          ORC_COEF_STATE: the flush writes C from the new state */
    double coef_ridge; /* ORC_COEF_STATE: ridge relative to the mean Gram eigenvalue */
    int pullback;      /* the sketched read's effective query: ORC_PULLBACK_SERIAL, _WY, or
                          _PROJ (the WY coefficients with projected per-slot factors) */
} orc_layer;

/* n independent tiles; every array is indexed by tile first. */
typedef struct {
    int n;
    const int* rank;     /* [n] sketch rank of the tile's head */
    double* S;           /* [n][dk][dv] stored state */
    double* U;           /* [n][rmax][dv] stored sketch, row j = u_j = S^T p_j */
    const double* Pt;    /* [n][rmax][dk] row j = column j of P_h (basis) */
    double* C;           /* [n][rmax][dk] row j = row j of the tile's coefficient map
                            (written by the flush in ORC_COEF_STATE mode) */
    const double* A;     /* [n] Mamba-2 A_h (unused otherwise) */
    double* rk;          /* [n][W][dk] ring keys */
    double* rv;          /* [n][W][dv] ring values */
    double* rg;          /* [n][W] (Mamba-2 dt, GDN alpha) or [n][W][dk] (KDA g) */
    double* rb;          /* [n][W] GDN/KDA beta (unused for Mamba-2) */
    int* count;          /* [n] entries buffered since the last flush */
    double* Sc;          /* [n][dk][dv] state copy of dense-fallback tiles (rank 0), stored
                            in the sketch dtype; may be NULL when no tile has rank 0 */
    double* rp;          /* [n][W][rmax] ORC_PULLBACK_PROJ: the ring's projected factors
                            C (Gamma_s (.) k_s), stored at the state's precision; may be
                            NULL otherwise */
} orc_tiles;

typedef struct {
    const double* q;     /* [n][dk] */
    const double* k;     /* [n][dk] */
    const double* v;     /* [n][dv] */
    const double* g;     /* [n] or [n][dk] (KDA) */
    const double* b;     /* [n] (GDN/KDA) */
    double* o;           /* [n][dv] */
} orc_step;

static int g_mutation = 0;
void orc_set_mutation(int m) { g_mutation = m; }

/* ------------------------------------------------------------ rounding */
static double round_f32(double x) { return (double)(float)x; }

static double round_bf16(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double store(int mode, double x) {
    if (mode == ORC_STORE_F32) return round_f32(x);
    if (mode == ORC_STORE_BF16) return round_bf16(x);
    return x;
}

static int gate_len(const orc_layer* L) { return L->family == ORC_KDA ? L->dk : 1; }

static double dot(const double* x, const double* y, int n) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += x[i] * y[i];
    return s;
}

/* Mamba-2 scalar decay a = exp(-dt * exp(A)). */
static double m2_decay(double dt, double A) { return exp(-dt * exp(A)); }

/* Write scale of B = s k v^T: dt for Mamba-2, beta for GDN/KDA. */
static double write_scale(const orc_layer* L, const double* g, double beta) {
    if (L->family == ORC_MAMBA2) return g_mutation == 8 ? 1.0 : g[0];
    return beta;
}

/* S <- M S + s k v^T for one entry (k, v, gate g, beta), S is dk x dv. */
static void apply_update(const orc_layer* L, double A, double* S,
                         const double* k, const double* v, const double* g,
                         double beta) {
    const int dk = L->dk, dv = L->dv;
    const double s = write_scale(L, g, beta);
    if (L->family == ORC_MAMBA2) {
        const double a = m2_decay(g[0], A);
        for (int m = 0; m < dk; ++m)
            for (int n = 0; n < dv; ++n) S[m * dv + n] = a * S[m * dv + n];
    } else {
        /* M S with M = alpha (I - beta k k^T) (GDN) or (I - beta k k^T) Diag(g) (KDA) */
        const double esign = (g_mutation == 2) ? -1.0 : 1.0;
        if (L->family == ORC_KDA && g_mutation != 6)
            for (int m = 0; m < dk; ++m)
                for (int n = 0; n < dv; ++n) S[m * dv + n] *= g[m];
        double* kS = (double*)malloc(sizeof(double) * dv);   /* k^T S */
        for (int n = 0; n < dv; ++n) {
            double t = 0.0;
            for (int m = 0; m < dk; ++m) t += k[m] * S[m * dv + n];
            kS[n] = t;
        }
        for (int m = 0; m < dk; ++m)
            for (int n = 0; n < dv; ++n)
                S[m * dv + n] -= esign * beta * k[m] * kS[n];
        free(kS);
        if (L->family == ORC_KDA && g_mutation == 6)
            for (int m = 0; m < dk; ++m)
                for (int n = 0; n < dv; ++n) S[m * dv + n] *= g[m];
        if (L->family == ORC_GDN)
            for (int m = 0; m < dk; ++m)
                for (int n = 0; n < dv; ++n) S[m * dv + n] *= g[0];
    }
    for (int m = 0; m < dk; ++m)
        for (int n = 0; n < dv; ++n) S[m * dv + n] += s * k[m] * v[n];
}

/* r <- M^T r for one entry: Mamba-2 a r; GDN alpha (r - beta (k.r) k);
 * KDA g (.) (r - beta (k.r) k). */
static void pull_back(const orc_layer* L, double A, double* r, const double* k,
                      const double* g, double beta) {
    const int dk = L->dk;
    if (g_mutation == 5) {
        if (L->family == ORC_MAMBA2) return;
    }
    if (L->family == ORC_MAMBA2) {
        const double a = m2_decay(g[0], A);
        for (int m = 0; m < dk; ++m) r[m] *= a;
        return;
    }
    const double d = dot(k, r, dk);
    for (int m = 0; m < dk; ++m) r[m] -= beta * d * k[m];
    if (g_mutation == 5) return;
    if (L->family == ORC_GDN)
        for (int m = 0; m < dk; ++m) r[m] *= g[0];
    else
        for (int m = 0; m < dk; ++m) r[m] *= g[m];
}

/* o = S^T x, S dk x dv. */
static void state_read(const orc_layer* L, const double* S, const double* x, double* o) {
    for (int n = 0; n < L->dv; ++n) {
        double t = 0.0;
        for (int m = 0; m < L->dk; ++m) t += S[m * L->dv + n] * x[m];
        o[n] = t;
    }
}

/* Tile accessors. */
#define TS(T, L, i) ((T)->S + (size_t)(i) * (L)->dk * (L)->dv)
#define TU(T, L, i) ((T)->U + (size_t)(i) * (L)->rmax * (L)->dv)
#define TP(T, L, i) ((T)->Pt + (size_t)(i) * (L)->rmax * (L)->dk)
#define TC(T, L, i) ((T)->C + (size_t)(i) * (L)->rmax * (L)->dk)
#define RK(T, L, i, s) ((T)->rk + ((size_t)(i) * (L)->W + (s)) * (L)->dk)
#define RV(T, L, i, s) ((T)->rv + ((size_t)(i) * (L)->W + (s)) * (L)->dv)
#define RG(T, L, i, s) ((T)->rg + ((size_t)(i) * (L)->W + (s)) * gate_len(L))
#define RB(T, L, i, s) ((T)->rb ? (T)->rb[(size_t)(i) * (L)->W + (s)] : 0.0)
#define RP(T, L, i, s) ((T)->rp + ((size_t)(i) * (L)->W + (s)) * (L)->rmax)

static double tile_A(const orc_tiles* T, int i) { return T->A ? T->A[i] : 0.0; }

/* Append the step's (k, v, gate, beta) of tile i at ring slot count. */
static void ring_append(const orc_layer* L, orc_tiles* T, const orc_step* st, int i) {
    const int slot = T->count[i];
    memcpy(RK(T, L, i, slot), st->k + (size_t)i * L->dk, sizeof(double) * L->dk);
    memcpy(RV(T, L, i, slot), st->v + (size_t)i * L->dv, sizeof(double) * L->dv);
    memcpy(RG(T, L, i, slot), st->g + (size_t)i * gate_len(L), sizeof(double) * gate_len(L));
    if (T->rb) T->rb[(size_t)i * L->W + slot] = st->b ? st->b[i] : 0.0;
    T->count[i] = slot + 1;
}

/* Pull the query back through ring entries n-1..0 (newest first): for each
 * entry, d = k.r contributes s d v to the buffered output, then r <- M^T r.
 * On return r = q~ (so that the state term is S0^T q~) and obuf holds the
 * exact contribution of the buffered updates. */
static void effective_query(const orc_layer* L, const orc_tiles* T, int i, int n,
                            const double* q, double* r, double* obuf) {
    const double A = tile_A(T, i);
    memcpy(r, q, sizeof(double) * L->dk);
    for (int j = 0; j < L->dv; ++j) obuf[j] = 0.0;
    for (int t = 0; t < n; ++t) {
        const int s = (g_mutation == 3) ? t : n - 1 - t;
        const double* k = RK(T, L, i, s);
        const double* g = RG(T, L, i, s);
        const double beta = RB(T, L, i, s);
        const double d = dot(k, r, L->dk);
        const double w = write_scale(L, g, beta) * d;
        const double* v = RV(T, L, i, s);
        for (int j = 0; j < L->dv; ++j) obuf[j] += w * v[j];
        pull_back(L, A, r, k, g, beta);
    }
}

/* Decay of buffered slot p at key element m: Mamba-2 a_p, GDN alpha_p,
 * KDA g_p[m]. */
static double slot_decay(const orc_layer* L, const orc_tiles* T, int i, int p, int m) {
    const double* g = RG(T, L, i, p);
    if (L->family == ORC_MAMBA2) return m2_decay(g[0], tile_A(T, i));
    return L->family == ORC_KDA ? g[m] : g[0];
}

/* The same q~ and o_buf as effective_query, with every buffered slot's
 * coefficient found at once (paper App. C.1).  Slots 0..n-1, oldest first.
 * Write D(j,l) = prod_{p=j+1..l} of the slot decays (elementwise for KDA;
 * the empty product is 1) and e = 1 for the erase terms of GDN/KDA (0 for
 * Mamba-2).  The serial form's coefficients d_j = k_j . r_j, r_j the query
 * pulled back through the slots newer than j, satisfy
 *     d_j + sum_{l>j} e beta_l <k_j, D(j,l) k_l> d_l = <k_j, D(j,n-1) q>,
 * an upper-triangular system solved by back substitution; then
 *     q~    = D(-1,n-1) q - sum_l e beta_l d_l D(-1,l) k_l,
 *     o_buf = sum_l s_l d_l v_l   (s_l the slot's write scale). */
static void effective_query_wy(const orc_layer* L, const orc_tiles* T, int i, int n,
                               const double* q, double* r, double* obuf, double* dcoef) {
    const int dk = L->dk;
    const int erase = L->family != ORC_MAMBA2;
    double* Lm = (double*)calloc((size_t)(n > 0 ? n : 1) * (n > 0 ? n : 1), sizeof(double));
    double* b = (double*)calloc(n > 0 ? n : 1, sizeof(double));
    double* d = (double*)calloc(n > 0 ? n : 1, sizeof(double));
    double* D = (double*)malloc(sizeof(double) * dk);
    for (int j = 0; j < n; ++j) {
        const double* kj = RK(T, L, i, j);
        for (int m = 0; m < dk; ++m) D[m] = (g_mutation == 15) ? slot_decay(L, T, i, j, m) : 1.0;
        for (int l = j + 1; l < n; ++l) {          /* D = D(j, l) */
            const double* kl = RK(T, L, i, l);
            double t = 0.0;
            for (int m = 0; m < dk; ++m) {
                D[m] *= slot_decay(L, T, i, l, m);
                t += kj[m] * D[m] * kl[m];
            }
            if (erase) Lm[(size_t)j * n + l] = RB(T, L, i, l) * t;
        }
        double t = 0.0;                              /* D = D(j, n-1) */
        for (int m = 0; m < dk; ++m) t += kj[m] * D[m] * q[m];
        b[j] = t;
    }
    for (int j = n - 1; j >= 0; --j) {
        double t = b[j];
        for (int l = j + 1; l < n; ++l) t -= Lm[(size_t)j * n + l] * d[l];
        d[j] = t;
    }
    for (int m = 0; m < dk; ++m) { D[m] = 1.0; r[m] = 0.0; }
    for (int l = 0; l < n; ++l) {                    /* D = D(-1, l) */
        const double* kl = RK(T, L, i, l);
        const double wl = erase ? RB(T, L, i, l) * d[l] : 0.0;
        for (int m = 0; m < dk; ++m) {
            D[m] *= slot_decay(L, T, i, l, m);
            r[m] -= wl * D[m] * kl[m];
        }
    }
    for (int m = 0; m < dk; ++m) r[m] += D[m] * q[m];
    for (int j = 0; j < L->dv; ++j) obuf[j] = 0.0;
    for (int l = 0; l < n; ++l) {
        const double w = write_scale(L, RG(T, L, i, l), RB(T, L, i, l)) * d[l];
        const double* v = RV(T, L, i, l);
        for (int j = 0; j < L->dv; ++j) obuf[j] += w * v[j];
    }
    if (dcoef)
        for (int l = 0; l < n; ++l) dcoef[l] = d[l];
    free(Lm); free(b); free(d); free(D);
}

/* The product of the decays of slots 0..s at key element m: D(-1, s) in
 * the notation above (Gamma_s). */
static double gamma_to(const orc_layer* L, const orc_tiles* T, int i, int s, int m) {
    double g = 1.0;
    for (int p = 0; p <= s; ++p) g *= slot_decay(L, T, i, p, m);
    return g;
}

/* Projected factor of ring slot s (paper App. C.2: the transition factors
 * projected through the fixed coefficient map, so that a slot keeps an
 * r-dimensional factor instead of a dk-dimensional one):
 *     P_s = C (Gamma_s (.) k_s),
 * with Gamma_s the product of the decays of slots 0..s (the decay part of
 * D(-1, s) in the triangular system above; a scalar for GDN, per channel
 * for KDA).  Formed when slot s is appended and stored at the state's
 * precision. */
static void project_slot(const orc_layer* L, orc_tiles* T, int i, int s) {
    const int r = T->rank[i];
    const double* k = RK(T, L, i, s);
    const double* C = TC(T, L, i);
    double* P = RP(T, L, i, s);
    for (int j = 0; j < r; ++j) {
        double t = 0.0;
        for (int m = 0; m < L->dk; ++m) {
            const double g = gamma_to(L, T, i, (g_mutation == 16 && s > 0) ? s - 1 : s, m);
            t += C[(size_t)j * L->dk + m] * g * k[m];
        }
        P[j] = store(L->state_store, t);
    }
}

/* c = C q~ from the projected factors (paper App. C.2): with the
 * coefficients d_l of the triangular system,
 *     q~ = Gamma_{n-1} (.) q - sum_l e beta_l d_l Gamma_l (.) k_l,
 * so  C q~ = C (Gamma_{n-1} (.) q) - sum_l e beta_l d_l P_l,
 * where only the first product touches a dk-dimensional vector. */
static void coef_projected(const orc_layer* L, const orc_tiles* T, int i, int n, const double* q,
                           const double* d, double* c) {
    const int r = T->rank[i];
    const int erase = L->family != ORC_MAMBA2;
    const double* C = TC(T, L, i);
    double* gq = (double*)malloc(sizeof(double) * L->dk);
    for (int m = 0; m < L->dk; ++m) gq[m] = gamma_to(L, T, i, n - 1, m) * q[m];
    for (int j = 0; j < r; ++j) {
        double t = dot(C + (size_t)j * L->dk, gq, L->dk);
        if (erase)
            for (int l = 0; l < n; ++l) t -= RB(T, L, i, l) * d[l] * RP(T, L, i, l)[j];
        c[j] = t;
    }
    free(gq);
}

/* Apply ring entries 0..n-1 in order to the fp64 copy S of the stored state. */
static void apply_ring(const orc_layer* L, const orc_tiles* T, int i, int n, double* S) {
    const double A = tile_A(T, i);
    for (int t = 0; t < n; ++t) {
        const int s = (g_mutation == 7) ? n - 1 - t : t;
        apply_update(L, A, S, RK(T, L, i, s), RV(T, L, i, s), RG(T, L, i, s), RB(T, L, i, s));
    }
}

static void store_state(const orc_layer* L, orc_tiles* T, int i, const double* S) {
    double* dst = TS(T, L, i);
    for (int e = 0; e < L->dk * L->dv; ++e) dst[e] = store(L->state_store, S[e]);
}

/* u_j = S^T p_j for the tile's r_h basis vectors. */
static void build_sketch(const orc_layer* L, orc_tiles* T, int i, const double* S) {
    const int r = T->rank[i];
    double* U = TU(T, L, i);
    const double* P = TP(T, L, i);
    double* u = (double*)malloc(sizeof(double) * L->dv);
    for (int j = 0; j < r; ++j) {
        state_read(L, S, P + (size_t)j * L->dk, u);
        for (int n = 0; n < L->dv; ++n) U[(size_t)j * L->dv + n] = store(L->sketch_store, u[n]);
    }
    free(u);
}

/* Dense-fallback tile: the updated state, stored in the sketch dtype. */
static void store_copy(const orc_layer* L, orc_tiles* T, int i, const double* S) {
    double* dst = T->Sc + (size_t)i * L->dk * L->dv;
    for (int e = 0; e < L->dk * L->dv; ++e) dst[e] = store(L->sketch_store, S[e]);
}

/* State-dependent coefficient map of tile i from its updated state S (dk x dv,
 * fp64) and the sketch rows u_j just stored (r x dv, as rounded at the store).
 * The non-flush read wants the coefficients c that best reproduce S^T q~ from
 * the stored sketch vectors, min_c |S^T q~ - sum_j c_j u_j|^2 (+ ridge), for
 * every q~; their normal equations give c = C q~ with
 *     G = [u_j . u_l]              the r x r Gram matrix of the sketch vectors,
 *     Y = [u_j . S[m, :]]          r x dk (the pages' U^T S0^T),
 *     (G + lambda I) C = Y,        lambda = ridge * trace(G) / r,
 * which is the pages' pseudoinverse form as ridge -> 0 when the u_j are
 * independent.  Solved by a Cholesky factorisation; C is stored in the
 * sketch dtype.  A zero sketch (trace 0) gives C = 0. */
static void build_coef_map(const orc_layer* L, orc_tiles* T, int i, const double* S,
                           const double* S_before) {
    const int r = T->rank[i], dk = L->dk, dv = L->dv;
    double* Cout = TC(T, L, i);
    const double* Uh = TU(T, L, i);
    double* u = NULL;
    if (g_mutation == 12) {                    /* planted: sketch before rounding */
        u = (double*)malloc(sizeof(double) * (size_t)r * dv);
        const double* P = TP(T, L, i);
        for (int j = 0; j < r; ++j) state_read(L, S, P + (size_t)j * dk, u + (size_t)j * dv);
        Uh = u;
    }
    const double* Sy = (g_mutation == 13) ? S_before : S;   /* planted: old state */
    double* G = (double*)malloc(sizeof(double) * (size_t)r * r);
    double* Y = (double*)malloc(sizeof(double) * (size_t)r * dk);
    double tr = 0.0;
    for (int j = 0; j < r; ++j) {
        for (int l = 0; l < r; ++l) G[j * r + l] = dot(Uh + (size_t)j * dv, Uh + (size_t)l * dv, dv);
        tr += G[j * r + j];
        for (int m = 0; m < dk; ++m) Y[(size_t)j * dk + m] = dot(Uh + (size_t)j * dv, Sy + (size_t)m * dv, dv);
    }
    if (tr == 0.0) {
        for (int e = 0; e < r * dk; ++e) Cout[e] = 0.0;
    } else {
        const double lambda = (g_mutation == 11) ? 0.0 : L->coef_ridge * tr / r;
        for (int j = 0; j < r; ++j) G[j * r + j] += lambda;
        /* G = R R^T, R lower triangular, written over the lower half of G */
        for (int j = 0; j < r; ++j) {
            double d = G[j * r + j];
            for (int l = 0; l < j; ++l) d -= G[j * r + l] * G[j * r + l];
            d = sqrt(d);
            G[j * r + j] = d;
            for (int t = j + 1; t < r; ++t) {
                double x = G[t * r + j];
                for (int l = 0; l < j; ++l) x -= G[t * r + l] * G[j * r + l];
                G[t * r + j] = x / d;
            }
        }
        /* every column of Y: solve R z = y, then R^T c = z */
        for (int m = 0; m < dk; ++m) {
            for (int j = 0; j < r; ++j) {
                double x = Y[(size_t)j * dk + m];
                for (int l = 0; l < j; ++l) x -= G[j * r + l] * Y[(size_t)l * dk + m];
                Y[(size_t)j * dk + m] = x / G[j * r + j];
            }
            for (int j = r - 1; j >= 0; --j) {
                double x = Y[(size_t)j * dk + m];
                for (int l = j + 1; l < r; ++l) x -= G[l * r + j] * Y[(size_t)l * dk + m];
                Y[(size_t)j * dk + m] = x / G[j * r + j];
            }
        }
        for (int e = 0; e < r * dk; ++e) Cout[e] = store(L->sketch_store, Y[e]);
    }
    free(G);
    free(Y);
    free(u);
}

static void write_out(const orc_layer* L, const orc_step* st, int i, const double* o) {
    for (int n = 0; n < L->dv; ++n) st->o[(size_t)i * L->dv + n] = store(L->out_store, o[n]);
}

/* ------------------------------------------------------------------ API */

/* Standard full-state step: S <- M S + B, o = S^T q, store S and o. */
int orc_full_step(const orc_layer* L, orc_tiles* T, const orc_step* st) {
    const size_t sz = (size_t)L->dk * L->dv;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < T->n; ++i) {
        double* S = (double*)malloc(sizeof(double) * sz);
        double* o = (double*)malloc(sizeof(double) * L->dv);
        memcpy(S, TS(T, L, i), sizeof(double) * sz);
        apply_update(L, tile_A(T, i), S, st->k + (size_t)i * L->dk, st->v + (size_t)i * L->dv,
                     st->g + (size_t)i * gate_len(L), st->b ? st->b[i] : 0.0);
        state_read(L, S, st->q + (size_t)i * L->dk, o);
        store_state(L, T, i, S);
        write_out(L, st, i, o);
        free(S);
        free(o);
    }
    return ORC_OK;
}

/* Flush: for every tile with count == W (or every tile, all != 0), apply the
 * count buffered entries to the state in order, store the state, build the
 * sketch from the updated state, write the exact output S^T q when a step is
 * given, and empty the ring. */
int orc_flush(const orc_layer* L, orc_tiles* T, const orc_step* st, int all) {
    const size_t sz = (size_t)L->dk * L->dv;
    int err = ORC_OK;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int i = 0; i < T->n; ++i) {
        const int n = T->count[i];
        if (n < 0 || n > L->W) { err |= ORC_ERR_COUNT; continue; }
        if (!all && n != L->W) continue;
        double* S = (double*)malloc(sizeof(double) * sz);
        double* o = (double*)malloc(sizeof(double) * L->dv);
        double* S0 = (double*)malloc(sizeof(double) * sz);
        memcpy(S, TS(T, L, i), sizeof(double) * sz);
        memcpy(S0, S, sizeof(double) * sz);
        apply_ring(L, T, i, n, S);
        store_state(L, T, i, S);
        if (T->rank[i] == 0) {
            store_copy(L, T, i, S);
        } else {
            build_sketch(L, T, i, S);
            if (L->coef_mode == ORC_COEF_STATE) build_coef_map(L, T, i, S, S0);
        }
        if (st && st->o) {
            state_read(L, g_mutation == 10 ? S0 : S, st->q + (size_t)i * L->dk, o);
            write_out(L, st, i, o);
        }
        T->count[i] = 0;
        free(S);
        free(S0);
        free(o);
    }
    return err;
}

/* Sketched read (non-flush step): append the step's entry; if the window is
 * not yet full, o = U (C q~) + o_buf from the stored sketch (a dense-fallback
 * tile: o = Sc^T q~ + o_buf from its stored state copy).  When the
 * append fills the window (count == W) no output is written here: the flush
 * produces it. */
int orc_read(const orc_layer* L, orc_tiles* T, const orc_step* st) {
    int err = ORC_OK;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int i = 0; i < T->n; ++i) {
        if (T->count[i] < 0 || T->count[i] >= L->W) { err |= ORC_ERR_COUNT; continue; }
        ring_append(L, T, st, i);
        const int n = T->count[i];
        if (n == L->W) continue;
        const int r = T->rank[i];
        double* qt = (double*)malloc(sizeof(double) * L->dk);
        double* obuf = (double*)malloc(sizeof(double) * L->dv);
        double* c = (double*)malloc(sizeof(double) * (r > 0 ? r : 1));
        double* o = (double*)malloc(sizeof(double) * L->dv);
        const double* q = st->q + (size_t)i * L->dk;
        double* dco = NULL;
        if (L->pullback == ORC_PULLBACK_PROJ) {
            project_slot(L, T, i, n - 1);              /* the appended slot's factor */
            dco = (double*)malloc(sizeof(double) * n);
        }
        if (L->pullback == ORC_PULLBACK_WY || L->pullback == ORC_PULLBACK_PROJ)
            effective_query_wy(L, T, i, n, q, qt, obuf, dco);
        else
            effective_query(L, T, i, n, q, qt, obuf);
        const double* C = TC(T, L, i);
        const double* U = TU(T, L, i);
        if (dco) {                    /* c = C q~ from the projected factors */
            coef_projected(L, T, i, n, q, dco, c);
            free(dco);
        } else {
            for (int j = 0; j < r; ++j)   /* c = C q~ */
                c[j] = dot(C + (size_t)j * L->dk, g_mutation == 9 ? q : qt, L->dk);
        }
        if (r == 0)                   /* dense fallback: o = Sc^T q~ + o_buf */
            state_read(L, T->Sc + (size_t)i * L->dk * L->dv, g_mutation == 14 ? q : qt, o);
        for (int n2 = 0; n2 < L->dv; ++n2) {  /* o = U c + o_buf */
            double t = (g_mutation == 1) ? 0.0 : obuf[n2];
            if (r == 0) t += o[n2];
            for (int j = 0; j < r; ++j) {
                const int jj = (g_mutation == 4) ? (j + 1) % r : j;
                t += U[(size_t)jj * L->dv + n2] * c[j];
            }
            o[n2] = t;
        }
        write_out(L, st, i, o);
        free(qt); free(obuf); free(c); free(o);
    }
    return err;
}

/* ReplaySSM step: append; before the window fills, o = S0^T q~ + o_buf read
 * from the full stored state; when it fills, apply the W entries, store the
 * state, o = S^T q from the updated state, and empty the ring. */
int orc_replay_step(const orc_layer* L, orc_tiles* T, const orc_step* st) {
    const size_t sz = (size_t)L->dk * L->dv;
    int err = ORC_OK;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int i = 0; i < T->n; ++i) {
        if (T->count[i] < 0 || T->count[i] >= L->W) { err |= ORC_ERR_COUNT; continue; }
        ring_append(L, T, st, i);
        const int n = T->count[i];
        double* o = (double*)malloc(sizeof(double) * L->dv);
        const double* q = st->q + (size_t)i * L->dk;
        if (n < L->W) {
            double* qt = (double*)malloc(sizeof(double) * L->dk);
            double* obuf = (double*)malloc(sizeof(double) * L->dv);
            effective_query(L, T, i, n, q, qt, obuf);
            state_read(L, TS(T, L, i), qt, o);
            if (g_mutation != 1)
                for (int j = 0; j < L->dv; ++j) o[j] += obuf[j];
            free(qt); free(obuf);
        } else {
            double* S = (double*)malloc(sizeof(double) * sz);
            memcpy(S, TS(T, L, i), sizeof(double) * sz);
            apply_ring(L, T, i, n, S);
            store_state(L, T, i, S);
            state_read(L, S, q, o);
            T->count[i] = 0;
            free(S);
        }
        write_out(L, st, i, o);
        free(o);
    }
    return err;
}

int orc_abi_version(void) { return 4; }

#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
void orc_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }
#else
int orc_num_threads(void) { return 1; }
void orc_set_num_threads(int n) { (void)n; }
#endif
