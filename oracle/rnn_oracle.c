/*
 * rnn_oracle.c -- plain, slow CPU oracle for the ONNX recurrent operators
 * RNN, GRU and LSTM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library, and it never calls it.
 *
 * What it computes is the exact-mode definition written out, in binary32 with
 * round-to-nearest-even, one rounding per written operation and no fused
 * multiply-add (the file is compiled with -ffp-contract=off and without any
 * fast-math option).  Sources, all on the onemodel page "Recurrent operators:
 * RNN, GRU, LSTM" unless stated otherwise:
 *   - gate packing of W, R, B and P ............ section "Support"
 *   - projection, recurrent product, gate loops .. section "Computation"
 *   - activation names, defaults, cursors ........ section "Activations"
 *   - sequence_lens, layout 1, omitted inputs,
 *     zero-size, hidden_size ..................... section "Choices the
 *                                                  specification leaves open"
 *   - NaN written as 0x7FC00000 .................. section "Exact mode"
 *   - scratch limit (Unsupported at plan time) ... section "Limits"
 *
 * Readings where the pages are silent or garbled:
 *   - Sigmoid, Tanh, ScaledTanh, Elu and Softplus are evaluated whole in
 *     binary64 from the binary32 argument and rounded once to binary32 (the
 *     library's own polynomials are not available).  The binary64 functions
 *     follow a fixed written method (below, "Binary64 elementary functions"),
 *     a fixed sequence of IEEE operations, so that an independent
 *     implementation performing the same operations gets the same bits.
 *   - clip <= 0 (or NaN) clamps nothing: clip acts only when given and positive.
 *   - A wrong activation count or an unknown name is InvalidInput; surplus
 *     alpha/beta values are ignored.
 *   - The optional bf16 projection rounds X and W to bfloat16 (RNE) and then
 *     runs the same fp32 accumulation; every product is exact in binary32.
 *
 * Data layout: dense row-major float32 in the ONNX shapes of the attribute
 * `layout`; sequence_lens is int32 on the host.  Every pointer is a host
 * pointer owned by the caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_OK = 0, ORC_INVALID_INPUT = 1, ORC_UNSUPPORTED = 2, ORC_NO_MEMORY = 4 };
enum { ORC_RNN = 0, ORC_GRU = 1, ORC_LSTM = 2 };

enum {
    ACT_SIGMOID = 0, ACT_TANH, ACT_RELU, ACT_AFFINE, ACT_LEAKYRELU,
    ACT_THRESHOLDEDRELU, ACT_SCALEDTANH, ACT_HARDSIGMOID, ACT_ELU,
    ACT_SOFTSIGN, ACT_SOFTPLUS, ACT_COUNT
};

typedef struct {
    int32_t kind;
    float alpha;
    float beta;
} orc_act;

typedef struct {
    int32_t op;                      /* ORC_RNN / ORC_GRU / ORC_LSTM */
    const char *direction;           /* "forward" | "reverse" | "bidirectional"; NULL = forward */
    int64_t hidden_size;             /* 0 = attribute absent */
    int32_t layout;                  /* 0 or 1 */
    int32_t n_activations;
    const char *const *activations;  /* NULL / 0 = defaults */
    int32_t n_alpha;
    const float *alpha;
    int32_t n_beta;
    const float *beta;
    int32_t has_clip;
    float clip;
    int32_t input_forget;            /* LSTM only */
    int32_t linear_before_reset;     /* GRU only */
    int32_t proj_bf16;               /* round X and W to bfloat16 before the projection */
    int32_t constant_weights;        /* only changes the scratch-limit sum */
} orc_attrs;

static const char *const ACT_NAMES[ACT_COUNT] = {
    "sigmoid", "tanh", "relu", "affine", "leakyrelu", "thresholdedrelu",
    "scaledtanh", "hardsigmoid", "elu", "softsign", "softplus"};

static void set_err(char *err, size_t errlen, const char *msg)
{
    if (err && errlen) {
        strncpy(err, msg, errlen - 1);
        err[errlen - 1] = 0;
    }
}

/* ---------------------------------------------------------------------- */
/* Binary64 elementary functions                                           */
/* ---------------------------------------------------------------------- */
/* The method (a reading; the pages name a polynomial document that is not
 * available).  Every step is one IEEE binary64 operation, rounded to
 * nearest, in the order written; no fused multiply-add.
 *   e^x      x NaN -> x; x > 708 -> +inf; x < -708 -> +0.  Otherwise Cody and
 *            Waite's reduction: k = rint(x * (1/ln 2)), r = (x - k*LN2_HI) -
 *            k*LN2_LO with ln 2 = LN2_HI + LN2_LO (LN2_HI has 32 trailing zero
 *            bits, so k*LN2_HI is exact); p = sum_{i=0..13} r^i / i! by
 *            Horner's rule from i = 13 down; result p * 2^k.
 *   e^x - 1  |x| < 1/2: x * (sum_{i=1..17} x^(i-1) / i!) by Horner's rule
 *            from i = 17 down; otherwise e^x - 1.
 *   tanh x   x NaN -> x; |x| > 22 -> copysign(1, x); otherwise
 *            m = e^(2|x|) - 1 (as above) and copysign(m / (m + 2), x).
 *   log(1+u) for 0 <= u <= 1: s = u / (2 + u), q = s*s,
 *            2 * s * (sum_{n=0..20} q^n / (2n + 1)) by Horner's rule from
 *            n = 20 down (the series of 2 atanh s).
 * Truncation errors are below 1e-17 relative in each range. */
static const double LN2_HI = 6.93147180369123816490e-01;   /* 0x3FE62E42FEE00000 */
static const double LN2_LO = 1.90821492927058770002e-10;   /* 0x3DEA39EF35793C76 */
static const double INV_LN2 = 1.44269504088896338700e+00;  /* 0x3FF71547652B82FE */

static double fact_inv(int i)                 /* 1 / i!, rounded once */
{
    double f = 1.0;
    for (int j = 2; j <= i; j++)
        f = f * (double)j;                     /* exact: i! < 2^53 for i <= 18 */
    return 1.0 / f;
}

static double orc_exp(double x)
{
    if (x != x)
        return x;
    if (x > 708.0)
        return INFINITY;
    if (x < -708.0)
        return 0.0;
    double k = rint(x * INV_LN2);
    double r = (x - k * LN2_HI) - k * LN2_LO;
    double p = fact_inv(13);
    for (int i = 12; i >= 0; i--)
        p = p * r + fact_inv(i);
    return ldexp(p, (int)k);
}

static double orc_expm1(double x)
{
    if (fabs(x) < 0.5) {
        double p = fact_inv(17);
        for (int i = 16; i >= 1; i--)
            p = p * x + fact_inv(i);
        return x * p;
    }
    return orc_exp(x) - 1.0;
}

static double orc_tanh(double x)
{
    if (x != x)
        return x;
    double ax = fabs(x);
    if (ax > 22.0)
        return copysign(1.0, x);
    double m = orc_expm1(2.0 * ax);
    return copysign(m / (m + 2.0), x);
}

static double orc_log1p01(double u)            /* 0 <= u <= 1 */
{
    double s = u / (2.0 + u);
    double q = s * s;
    double p = 1.0 / 41.0;
    for (int n = 19; n >= 0; n--)
        p = p * q + 1.0 / (double)(2 * n + 1);
    return 2.0 * s * p;
}

/* ---------------------------------------------------------------------- */
/* Activations ("Activations", definitions paragraph)                      */
/* ---------------------------------------------------------------------- */

float orc_activation(int32_t kind, float alpha, float beta, float x)
{
    switch (kind) {
    case ACT_SIGMOID:
        return (float)(1.0 / (1.0 + orc_exp(-(double)x)));
    case ACT_TANH:
        return (float)orc_tanh((double)x);
    case ACT_RELU:                       /* keeps a NaN (and -0) */
        return x < 0.0f ? 0.0f : x;
    case ACT_AFFINE: {
        float ax = alpha * x;
        return ax + beta;
    }
    case ACT_LEAKYRELU:
        return x < 0.0f ? alpha * x : x;
    case ACT_THRESHOLDEDRELU:
        return x > alpha ? x : 0.0f;
    case ACT_SCALEDTANH:
        return (float)((double)alpha * orc_tanh((double)beta * (double)x));
    case ACT_HARDSIGMOID: {
        float ax = alpha * x;
        float y = ax + beta;
        y = y < 0.0f ? 0.0f : y;        /* max(0, .) that lets a NaN through */
        y = y > 1.0f ? 1.0f : y;        /* min(1, .) likewise */
        return y;
    }
    case ACT_ELU:
        return x >= 0.0f ? x : (float)((double)alpha * orc_expm1((double)x));
    case ACT_SOFTSIGN: {
        float den = 1.0f + fabsf(x);
        return x / den;
    }
    case ACT_SOFTPLUS:
        if (x > 20.0f)                  /* log(1 + e^x) rounds to x */
            return x;
        if (x > 0.0f)                   /* x + log(1 + e^-x) */
            return (float)((double)x + orc_log1p01(orc_exp(-(double)x)));
        return (float)orc_log1p01(orc_exp((double)x));   /* NaN passes through */
    default:
        return NAN;
    }
}

static int name_to_kind(const char *name)
{
    char low[32];
    size_t n = strlen(name);
    if (n == 0 || n >= sizeof(low))
        return -1;
    for (size_t i = 0; i <= n; i++) {
        char ch = name[i];
        low[i] = (ch >= 'A' && ch <= 'Z') ? (char)(ch - 'A' + 'a') : ch;
    }
    for (int k = 0; k < ACT_COUNT; k++)
        if (strcmp(low, ACT_NAMES[k]) == 0)
            return k;
    return -1;
}

static int takes_alpha(int k)
{
    return k == ACT_AFFINE || k == ACT_SCALEDTANH || k == ACT_HARDSIGMOID ||
           k == ACT_LEAKYRELU || k == ACT_THRESHOLDEDRELU || k == ACT_ELU;
}

static int takes_beta(int k)
{
    return k == ACT_AFFINE || k == ACT_SCALEDTANH || k == ACT_HARDSIGMOID;
}

static float default_alpha(int k)
{
    switch (k) {
    case ACT_LEAKYRELU: return 0.01f;
    case ACT_THRESHOLDEDRELU: return 1.0f;
    case ACT_ELU: return 1.0f;
    case ACT_HARDSIGMOID: return 0.2f;
    case ACT_AFFINE: return 1.0f;
    case ACT_SCALEDTANH: return 1.0f;
    default: return 0.0f;
    }
}

static float default_beta(int k)
{
    switch (k) {
    case ACT_HARDSIGMOID: return 0.5f;
    case ACT_AFFINE: return 0.0f;
    case ACT_SCALEDTANH: return 0.0f;
    default: return 0.0f;
    }
}

static int gates_of(int op) { return op == ORC_LSTM ? 4 : op == ORC_GRU ? 3 : 1; }

/*
 * Resolve f, g, h for each direction.  out[d * 3 + j] is activation j of
 * direction d.  The list may be absent (defaults), one set (both directions)
 * or, for a bidirectional layer, a forward set followed by a reverse set.
 * alpha and beta are walked with separate cursors in list order.
 */
int32_t orc_parse_activations(int32_t op, int32_t dirs, int32_t n_names,
                              const char *const *names, int32_t n_alpha,
                              const float *alpha, int32_t n_beta,
                              const float *beta, orc_act *out,
                              char *err, size_t errlen)
{
    int na = op == ORC_LSTM ? 3 : op == ORC_GRU ? 2 : 1;
    static const int defaults[3][3] = {
        {ACT_TANH, 0, 0},                          /* RNN  */
        {ACT_SIGMOID, ACT_TANH, 0},                /* GRU  */
        {ACT_SIGMOID, ACT_TANH, ACT_TANH}};        /* LSTM */
    memset(out, 0, sizeof(orc_act) * 6);
    if (n_names == 0 || names == NULL) {
        for (int d = 0; d < dirs; d++)
            for (int j = 0; j < na; j++) {
                int k = defaults[op][j];
                out[d * 3 + j].kind = k;
                out[d * 3 + j].alpha = default_alpha(k);
                out[d * 3 + j].beta = default_beta(k);
            }
        return ORC_OK;
    }
    if (!(n_names == na || (dirs == 2 && n_names == 2 * na))) {
        set_err(err, errlen, "activations: wrong number of entries");
        return ORC_INVALID_INPUT;
    }
    int ca = 0, cb = 0;
    orc_act parsed[6];
    for (int i = 0; i < n_names; i++) {
        if (names[i] == NULL) {
            set_err(err, errlen, "activations: null name");
            return ORC_INVALID_INPUT;
        }
        int k = name_to_kind(names[i]);
        if (k < 0) {
            set_err(err, errlen, "activations: unknown name");
            return ORC_INVALID_INPUT;
        }
        parsed[i].kind = k;
        parsed[i].alpha = default_alpha(k);
        parsed[i].beta = default_beta(k);
        if (takes_alpha(k) && ca < n_alpha)
            parsed[i].alpha = alpha[ca++];
        if (takes_beta(k) && cb < n_beta)
            parsed[i].beta = beta[cb++];
    }
    for (int d = 0; d < dirs; d++)
        for (int j = 0; j < na; j++)
            out[d * 3 + j] = (n_names == na) ? parsed[j] : parsed[d * na + j];
    return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* Small helpers                                                           */
/* ---------------------------------------------------------------------- */

static float canon(float v)
{
    if (v != v) {
        uint32_t bits = 0x7FC00000u;
        float q;
        memcpy(&q, &bits, sizeof q);
        return q;
    }
    return v;
}

/* binary32 -> bfloat16 -> binary32, round to nearest even; a NaN stays a quiet NaN. */
float orc_round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
        u = (u | 0x00400000u) & 0xFFFF0000u;
    } else {
        uint32_t lsb = (u >> 16) & 1u;
        u = u + 0x7FFFu + lsb;
        u &= 0xFFFF0000u;
    }
    float r;
    memcpy(&r, &u, sizeof r);
    return r;
}

static float clipv(float x, int on, float c)
{
    if (!on)
        return x;
    /* NaN passes through both compares */
    return x > c ? c : (x < -c ? -c : x);
}

/* ONNX index helpers for the two layouts ("layout = 1": batch-first). */
static size_t x_at(int layout, int64_t t, int64_t b, int64_t S, int64_t Bt, int64_t I)
{
    return layout == 0 ? (size_t)((t * Bt + b) * I) : (size_t)((b * S + t) * I);
}

static size_t y_at(int layout, int64_t t, int64_t d, int64_t b, int64_t S,
                   int64_t D, int64_t Bt, int64_t H)
{
    return layout == 0 ? (size_t)(((t * D + d) * Bt + b) * H)
                       : (size_t)(((b * S + t) * D + d) * H);
}

static size_t s_at(int layout, int64_t d, int64_t b, int64_t D, int64_t Bt, int64_t H)
{
    return layout == 0 ? (size_t)((d * Bt + b) * H) : (size_t)((b * D + d) * H);
}

/*
 * out[n] = sum_k a[k] * mt[k][n] for n in [0, ncols), with mt row-major of
 * row length ld.  One accumulator per output, k increasing from +0.0, each
 * product and each sum rounded separately (the shared-GEMM rule of the
 * "Computation" section, step 1).
 */
static void vec_mat(const float *a, int64_t K, const float *mt, int64_t ld,
                    int64_t ncols, float *out)
{
    for (int64_t n = 0; n < ncols; n++)
        out[n] = 0.0f;
    for (int64_t k = 0; k < K; k++) {
        const float ak = a[k];
        const float *row = mt + (size_t)k * ld;
        for (int64_t n = 0; n < ncols; n++) {
            float p = ak * row[n];
            out[n] = out[n] + p;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* The operator                                                            */
/* ---------------------------------------------------------------------- */

int32_t orc_run(const orc_attrs *at, int64_t S, int64_t Bt, int64_t I, int64_t H,
                int64_t D, const float *X, const float *W, const float *R,
                const float *B, const int32_t *lens, const float *h0,
                const float *c0, const float *P, float *Y, float *Yh, float *Yc,
                int32_t n_threads, char *err, size_t errlen)
{
    set_err(err, errlen, "");
    if (at == NULL) {
        set_err(err, errlen, "attrs is NULL");
        return ORC_INVALID_INPUT;
    }
    const int op = at->op;
    if (op != ORC_RNN && op != ORC_GRU && op != ORC_LSTM) {
        set_err(err, errlen, "unknown operator");
        return ORC_INVALID_INPUT;
    }
    const int G = gates_of(op);

    /* direction and number of directions */
    int reverse_only = 0, want_dirs = 1;
    if (at->direction == NULL || strcmp(at->direction, "forward") == 0) {
        want_dirs = 1;
    } else if (strcmp(at->direction, "reverse") == 0) {
        want_dirs = 1;
        reverse_only = 1;
    } else if (strcmp(at->direction, "bidirectional") == 0) {
        want_dirs = 2;
    } else {
        set_err(err, errlen, "direction: unknown value");
        return ORC_INVALID_INPUT;
    }
    if (D != want_dirs) {
        set_err(err, errlen, "num_directions does not match direction");
        return ORC_INVALID_INPUT;
    }
    if (at->layout != 0 && at->layout != 1) {
        set_err(err, errlen, "layout must be 0 or 1");
        return ORC_INVALID_INPUT;
    }
    if (S < 0 || Bt < 0 || I < 0 || H < 0) {
        set_err(err, errlen, "negative dimension");
        return ORC_INVALID_INPUT;
    }
    /* hidden_size: optional; equal to R's last dimension; zero is an error */
    if (H == 0) {
        set_err(err, errlen, "hidden size is zero");
        return ORC_INVALID_INPUT;
    }
    if (at->hidden_size != 0 && at->hidden_size != H) {
        set_err(err, errlen, "hidden_size does not match R");
        return ORC_INVALID_INPUT;
    }
    if (op != ORC_LSTM && (at->input_forget || c0 || P || Yc)) {
        set_err(err, errlen, "input_forget / initial_c / P / Y_c are LSTM-only");
        return ORC_INVALID_INPUT;
    }
    if (op != ORC_GRU && at->linear_before_reset) {
        set_err(err, errlen, "linear_before_reset is GRU-only");
        return ORC_INVALID_INPUT;
    }
    orc_act acts[6];
    int32_t st = orc_parse_activations(op, (int32_t)D, at->n_activations, at->activations,
                                       at->n_alpha, at->alpha, at->n_beta, at->beta,
                                       acts, err, errlen);
    if (st != ORC_OK)
        return st;

    /* scratch limit, per direction, in floats ("Limits") */
    {
        double need = (double)S * (double)Bt * (double)G * (double)H + 4.0 * (double)Bt * (double)H;
        if (!at->constant_weights)
            need += (double)G * (double)H * ((double)I + (double)H);
        if (!(need < 1073741824.0)) {
            set_err(err, errlen, "per-direction scratch reaches 2^30 floats");
            return ORC_UNSUPPORTED;
        }
    }
    if (lens)
        for (int64_t b = 0; b < Bt; b++)
            if (lens[b] < 0 || lens[b] > S) {
                set_err(err, errlen, "sequence_lens entry outside [0, seq]");
                return ORC_INVALID_INPUT;
            }

    const int layout = at->layout;
    const size_t nstate = (size_t)(D * Bt * H);

    /* zero-size: nothing runs; final states are the initial states or zeros */
    if (S == 0 || Bt == 0) {
        for (size_t i = 0; i < nstate; i++) {
            if (Yh)
                Yh[i] = canon(h0 ? h0[i] : 0.0f);
            if (Yc)
                Yc[i] = canon(c0 ? c0[i] : 0.0f);
        }
        return ORC_OK;
    }

    const int clip_on = at->has_clip && at->clip > 0.0f;
    const float C = at->clip;
    const int64_t GH = (int64_t)G * H;
    const int lbr = at->linear_before_reset;

    float *Wt = malloc(sizeof(float) * (size_t)(I * GH));
    float *Rt = malloc(sizeof(float) * (size_t)(H * GH));
    float *XW = malloc(sizeof(float) * (size_t)(S * Bt * GH));
    float *Xr = at->proj_bf16 ? malloc(sizeof(float) * (size_t)(S * Bt * I)) : NULL;
    if (!Wt || !Rt || !XW || (at->proj_bf16 && !Xr)) {
        free(Wt); free(Rt); free(XW); free(Xr);
        set_err(err, errlen, "out of host memory");
        return ORC_NO_MEMORY;
    }
    const float *Xuse = X;
    if (at->proj_bf16) {
        for (size_t i = 0; i < (size_t)(S * Bt * I); i++)
            Xr[i] = orc_round_bf16(X[i]);
        Xuse = Xr;
    }

    if (Y) {
        size_t ny = (size_t)(S * D * Bt * H);
        for (size_t i = 0; i < ny; i++)
            Y[i] = 0.0f;            /* positions t >= len_b stay +0.0 */
    }

    int nt = n_threads > 0 ? n_threads : 1;

    for (int64_t d = 0; d < D; d++) {
        const int reverse = reverse_only || d == 1;
        const orc_act *fa = &acts[d * 3];

        /* Transposition of W[d] and R[d] (exact). */
        const float *Wd = W + (size_t)(d * GH * I);
        const float *Rd = R + (size_t)(d * GH * H);
        for (int64_t n = 0; n < GH; n++)
            for (int64_t k = 0; k < I; k++) {
                float w = Wd[(size_t)(n * I + k)];
                Wt[(size_t)(k * GH + n)] = at->proj_bf16 ? orc_round_bf16(w) : w;
            }
        for (int64_t n = 0; n < GH; n++)
            for (int64_t k = 0; k < H; k++)
                Rt[(size_t)(k * GH + n)] = Rd[(size_t)(n * H + k)];

        /* Step 1: input projection of all time steps, XW[t][b][:] */
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t m = 0; m < S * Bt; m++) {
            int64_t t = m / Bt, b = m % Bt;
            vec_mat(Xuse + x_at(layout, t, b, S, Bt, I), I, Wt, GH, GH,
                    XW + (size_t)(m * GH));
        }

        const float *Wb = B ? B + (size_t)(d * 2 * GH) : NULL;
        const float *Rb = B ? B + (size_t)(d * 2 * GH + GH) : NULL;
        const float *Pd = P ? P + (size_t)(d * 3 * H) : NULL;

        /* Steps 2 and 3: rows are independent, so each row runs its own steps. */
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
        for (int64_t b = 0; b < Bt; b++) {
            float *h = malloc(sizeof(float) * (size_t)H);
            float *c = malloc(sizeof(float) * (size_t)H);
            float *hn = malloc(sizeof(float) * (size_t)H);
            float *cn = malloc(sizeof(float) * (size_t)H);
            float *rec = malloc(sizeof(float) * (size_t)GH);
            float *s = malloc(sizeof(float) * (size_t)H);
            float *rh = malloc(sizeof(float) * (size_t)H);
            float *zg = malloc(sizeof(float) * (size_t)H);
            size_t so = s_at(layout, d, b, D, Bt, H);
            for (int64_t u = 0; u < H; u++) {
                h[u] = h0 ? h0[so + u] : 0.0f;
                c[u] = c0 ? c0[so + u] : 0.0f;
            }
            const int64_t len = lens ? lens[b] : S;
            for (int64_t j = 0; j < len; j++) {
                const int64_t t = reverse ? len - 1 - j : j;
                const float *xw = XW + (size_t)((t * Bt + b) * GH);
                /* recurrent product for the whole gate width, or only the
                   z and r columns for GRU with linear_before_reset = 0 */
                int64_t ncols = (op == ORC_GRU && !lbr) ? 2 * H : GH;
                vec_mat(h, H, Rt, GH, ncols, rec);

                if (op == ORC_RNN) {
                    for (int64_t u = 0; u < H; u++) {
                        float pre = xw[u] + rec[u];
                        if (B) {
                            pre = pre + Wb[u];
                            pre = pre + Rb[u];
                        }
                        pre = clipv(pre, clip_on, C);
                        hn[u] = orc_activation(fa[0].kind, fa[0].alpha, fa[0].beta, pre);
                    }
                } else if (op == ORC_GRU) {
                    /* gate order z, r, h */
                    for (int64_t u = 0; u < H; u++) {
                        float pz = xw[u] + rec[u];
                        float pr = xw[H + u] + rec[H + u];
                        if (B) {
                            pz = pz + Wb[u];
                            pz = pz + Rb[u];
                            pr = pr + Wb[H + u];
                            pr = pr + Rb[H + u];
                        }
                        pz = clipv(pz, clip_on, C);
                        pr = clipv(pr, clip_on, C);
                        zg[u] = orc_activation(fa[0].kind, fa[0].alpha, fa[0].beta, pz);
                        float r = orc_activation(fa[0].kind, fa[0].alpha, fa[0].beta, pr);
                        if (!lbr)
                            s[u] = r * h[u];           /* r (.) H_prev, rounded */
                        else
                            rh[u] = r;                 /* keep r for the candidate */
                    }
                    if (!lbr)   /* second small product (r (.) H_prev) . Rh^T */
                        vec_mat(s, H, Rt + 2 * H, GH, H, rh);
                    for (int64_t u = 0; u < H; u++) {
                        float ph;
                        if (!lbr) {
                            ph = xw[2 * H + u] + rh[u];
                            if (B) {
                                ph = ph + Wb[2 * H + u];
                                ph = ph + Rb[2 * H + u];
                            }
                        } else {
                            float r = rh[u];
                            float inner = B ? rec[2 * H + u] + Rb[2 * H + u] : rec[2 * H + u];
                            float gated = r * inner;
                            ph = xw[2 * H + u] + gated;
                            if (B)
                                ph = ph + Wb[2 * H + u];
                        }
                        ph = clipv(ph, clip_on, C);
                        float ht = orc_activation(fa[1].kind, fa[1].alpha, fa[1].beta, ph);
                        float z = zg[u];
                        float omz = 1.0f - z;
                        float a1 = omz * ht;
                        float a2 = z * h[u];
                        hn[u] = a1 + a2;
                    }
                } else {
                    /* LSTM, gate order i, o, f, c; peepholes P in order i, o, f */
                    for (int64_t u = 0; u < H; u++) {
                        float pre[4];
                        for (int g = 0; g < 4; g++) {
                            float v = xw[g * H + u] + rec[g * H + u];
                            if (B) {
                                v = v + Wb[g * H + u];
                                v = v + Rb[g * H + u];
                            }
                            pre[g] = v;
                        }
                        float cp = c[u];
                        if (Pd) {
                            float pi = Pd[u] * cp;
                            float pf = Pd[2 * H + u] * cp;
                            pre[0] = pre[0] + pi;
                            pre[2] = pre[2] + pf;
                        }
                        float pi_ = clipv(pre[0], clip_on, C);
                        float pf_ = clipv(pre[2], clip_on, C);
                        float pc_ = clipv(pre[3], clip_on, C);
                        float ig = orc_activation(fa[0].kind, fa[0].alpha, fa[0].beta, pi_);
                        float fg = at->input_forget
                                       ? 1.0f - ig
                                       : orc_activation(fa[0].kind, fa[0].alpha, fa[0].beta, pf_);
                        float ct = orc_activation(fa[1].kind, fa[1].alpha, fa[1].beta, pc_);
                        float k1 = fg * cp;
                        float k2 = ig * ct;
                        float cnew = k1 + k2;
                        float po = pre[1];
                        if (Pd) {
                            float pov = Pd[H + u] * cnew;
                            po = po + pov;
                        }
                        po = clipv(po, clip_on, C);
                        float og = orc_activation(fa[0].kind, fa[0].alpha, fa[0].beta, po);
                        float hc = orc_activation(fa[2].kind, fa[2].alpha, fa[2].beta, cnew);
                        hn[u] = og * hc;
                        cn[u] = cnew;
                    }
                }
                if (Y) {
                    float *yo = Y + y_at(layout, t, d, b, S, D, Bt, H);
                    for (int64_t u = 0; u < H; u++)
                        yo[u] = canon(hn[u]);
                }
                for (int64_t u = 0; u < H; u++) {
                    h[u] = hn[u];
                    if (op == ORC_LSTM)
                        c[u] = cn[u];
                }
            }
            /* final states: after the last valid step; a row of length 0 gives 0 */
            for (int64_t u = 0; u < H; u++) {
                if (Yh)
                    Yh[so + u] = len == 0 ? 0.0f : canon(h[u]);
                if (Yc)
                    Yc[so + u] = len == 0 ? 0.0f : canon(c[u]);
            }
            free(h); free(c); free(hn); free(cn); free(rec); free(s); free(rh); free(zg);
        }
    }
    free(Wt);
    free(Rt);
    free(XW);
    free(Xr);
    return ORC_OK;
}

/* The projection alone, XW[d][m][n] with m in X's (t, b) order of layout 0;
 * exported so that a test can pin the shared-GEMM step by itself. */
int32_t orc_projection(int64_t M, int64_t I, int64_t N, const float *X,
                       const float *W, int32_t bf16, float *out, int32_t n_threads)
{
    float *Wt = malloc(sizeof(float) * (size_t)(I * N));
    float *xr = malloc(sizeof(float) * (size_t)(I > 0 ? I : 1) * (size_t)(M > 0 ? M : 1));
    if (!Wt || !xr) {
        free(Wt); free(xr);
        return ORC_NO_MEMORY;
    }
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < I; k++) {
            float w = W[(size_t)(n * I + k)];
            Wt[(size_t)(k * N + n)] = bf16 ? orc_round_bf16(w) : w;
        }
    for (size_t i = 0; i < (size_t)(M * I); i++)
        xr[i] = bf16 ? orc_round_bf16(X[i]) : X[i];
    int nt = n_threads > 0 ? n_threads : 1;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t m = 0; m < M; m++)
        vec_mat(xr + (size_t)(m * I), I, Wt, N, N, out + (size_t)(m * N));
    free(Wt);
    free(xr);
    return ORC_OK;
}
