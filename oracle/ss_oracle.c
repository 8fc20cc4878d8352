/*
 * ss_oracle.c -- float64 CPU oracle for the Mamba selective scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke entry and the bench's
 * cpu_baseline leg may load this library.  It shares no code, header, table
 * or constant with the HIP path: it is the plain definition of the method,
 * written out as a sequential loop in double precision, so that a reader can
 * check it against the pages by eye.
 *
 * Sources (page title, then section):
 *   "Mamba" (stanleyjacob.dev walkthrough), Part IV Stage 4: the zero-order
 *       hold for A, Abar = exp(Delta*A) elementwise (A diagonal), and the
 *       Euler rule Bbar = Delta*B; the recurrence h_t = Abar_t h_{t-1} +
 *       Bbar_t x_t with readout y_t = C_t h_t.
 *   same page, Part IV Stage 5: the operand shapes u, delta (B,D,L); A (D,N);
 *       B, C (B,N,L); D (D); z (B,D,L); delta_bias added to delta and the
 *       softplus applied inside the op when delta_softplus is set.
 *   same page, Part IV Stage 6: skip y = y + D*u, then the gate y*SiLU(z).
 *   same page, Part V "the hardware-aware scan kernel": the state starts at
 *       zero and the per-step loop order (discretize, update, read out).
 *   same page, Part IV Stage 7: the backward recomputes states and produces
 *       gradients for u, Delta, A, B, C, D and z.
 *   "mamba-metal" README, "Long-context prompts": the scan also returns the
 *       final state, from which single-token decode continues (step).
 *   "Mamba, on a laptop GPU", "The state lives in registers": gradients of
 *       B and C sum over channels.
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *   - softplus(x) = log(1 + e^x), evaluated in the overflow-safe form
 *     max(x,0) + log1p(e^{-|x|});
 *   - the bias is added to delta whether or not softplus is applied;
 *   - out = (sum_n C h + D u) * z * sigmoid(z): the D skip comes before the gate;
 *   - ragged rows: row b runs lengths[b] steps from a zero state (or h0),
 *     the outputs past that length are exactly 0 and the final state is the
 *     state after lengths[b] steps;
 *   - packed documents ("niverel-mamba" README, "seq_idx strict reset"):
 *     wherever seq_idx[b,t] differs from seq_idx[b,t-1] (t >= 1) the state
 *     is set to zero before step t, so every document starts from zero and a
 *     packed row equals its documents run one by one;
 *   - the loss for the backward is sum(dy * out) + sum(dlast * h_final);
 *     gradients of B and C sum over channels d, those of A, D and bias over
 *     batch rows and time; dh0 is the gradient of that loss w.r.t. the
 *     initial state.
 *
 * Everything is computed per channel (b, d) independently; threads split the
 * channels and never change the arithmetic of a channel.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* log(1 + e^x) without overflow for large x. */
static double softplus(double x)
{
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* 1 / (1 + e^{-x}) without overflow for large |x|. */
static double sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

typedef struct {
    int64_t batch, dim, dstate, seqlen;
    int softplus;
    const double *u, *delta, *A, *Bm, *Cm, *Dskip, *z, *bias, *h0, *dy;
    const int64_t *lengths;
    const int64_t *seq_idx; /* optional (B,L) document ids */
    const double *dlast;    /* optional (B,D,N) gradient w.r.t. the final state */
    double *dh0;            /* optional (B,D,N) gradient w.r.t. the initial state */
    const int64_t *rows; /* optional subset of channels b*dim+d */
    int64_t nrows;
    /* forward outputs */
    double *y, *last_state, *states;
    int64_t states_every;
    /* backward outputs */
    double *du, *ddelta, *dz, *dA, *dB, *dC, *dD, *dbias;
} job_t;

typedef struct {
    const job_t *job;
    int64_t first, last; /* [first, last) over the channel list */
    /* per-thread partial sums for the backward's reduced gradients */
    double *dA, *dB, *dC, *dD, *dbias;
} slice_t;

/* Step t of row b starts a new document: the state is reset to zero. */
static int resets(const job_t *j, int64_t b, int64_t t)
{
    const int64_t *s = j->seq_idx;
    return s != NULL && t > 0 && s[b * j->seqlen + t] != s[b * j->seqlen + t - 1];
}

static int64_t row_len(const job_t *j, int64_t b)
{
    int64_t len = j->lengths ? j->lengths[b] : j->seqlen;
    if (len < 0) len = 0;
    if (len > j->seqlen) len = j->seqlen;
    return len;
}

/* Forward of one channel (b, d): the sequential recurrence of Stage 4/5. */
static void forward_channel(const job_t *j, int64_t b, int64_t d)
{
    const int64_t D = j->dim, N = j->dstate, L = j->seqlen;
    const int64_t ch = b * D + d;
    const int64_t len = row_len(j, b);
    const double *u = j->u + ch * L, *dl = j->delta + ch * L;
    const double *zz = j->z ? j->z + ch * L : NULL;
    const double *Bb = j->Bm + b * N * L, *Cb = j->Cm + b * N * L;
    const double *Arow = j->A + d * N;
    const double bias = j->bias ? j->bias[d] : 0.0;
    double *y = j->y + ch * L;
    double h[64];

    for (int64_t n = 0; n < N; ++n)
        h[n] = j->h0 ? j->h0[ch * N + n] : 0.0;

    int64_t K = 0;
    if (j->states) {
        K = (L + j->states_every - 1) / j->states_every;
        for (int64_t n = 0; n < N; ++n)
            j->states[(ch * K + 0) * N + n] = h[n];
    }

    for (int64_t t = 0; t < len; ++t) {
        if (resets(j, b, t))                       /* a new document starts */
            for (int64_t n = 0; n < N; ++n)
                h[n] = 0.0;
        double x = dl[t] + bias;
        double dt = j->softplus ? softplus(x) : x;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double a = exp(dt * Arow[n]);          /* Abar = exp(Delta*A)   */
            double bb = dt * Bb[n * L + t];        /* Bbar = Delta*B        */
            h[n] = a * h[n] + bb * u[t];           /* h = Abar h + Bbar u   */
            acc += Cb[n * L + t] * h[n];           /* y = C h               */
        }
        if (j->Dskip)
            acc += j->Dskip[d] * u[t];             /* skip: + D u           */
        if (zz)
            acc *= zz[t] * sigmoid(zz[t]);         /* gate: * SiLU(z)       */
        y[t] = acc;
        if (j->states && (t + 1) % j->states_every == 0 && (t + 1) / j->states_every < K)
            for (int64_t n = 0; n < N; ++n)
                j->states[(ch * K + (t + 1) / j->states_every) * N + n] = h[n];
    }
    for (int64_t t = len; t < L; ++t)
        y[t] = 0.0;
    if (j->states)
        for (int64_t k = 1; k < K; ++k)
            if (k * j->states_every > len)
                for (int64_t n = 0; n < N; ++n)
                    j->states[(ch * K + k) * N + n] = h[n];
    if (j->last_state)
        for (int64_t n = 0; n < N; ++n)
            j->last_state[ch * N + n] = h[n];
}

/*
 * Backward of one channel: reverse-mode differentiation of forward_channel
 * for the loss sum_t dy_t * out_t + sum_n dlast[n] * h_final[n].  The
 * forward states are recomputed and kept for every step (Stage 7: the states
 * are recomputed, not stored by the forward).  g[n] carries dLoss/dh_t[n]
 * from step t+1 back to step t.  At a document start the carried state is
 * multiplied by keep = 0 (the reset), so nothing flows back through it.
 */
static void backward_channel(const slice_t *s, int64_t b, int64_t d, double *hist)
{
    const job_t *j = s->job;
    const int64_t D = j->dim, N = j->dstate, L = j->seqlen;
    const int64_t ch = b * D + d;
    const int64_t len = row_len(j, b);
    const double *u = j->u + ch * L, *dl = j->delta + ch * L;
    const double *zz = j->z ? j->z + ch * L : NULL;
    const double *Bb = j->Bm + b * N * L, *Cb = j->Cm + b * N * L;
    const double *Arow = j->A + d * N;
    const double bias = j->bias ? j->bias[d] : 0.0;
    const double Dd = j->Dskip ? j->Dskip[d] : 0.0;
    const double *dy = j->dy + ch * L;
    double g[64];

    /* hist[t*N + n] = h after t steps (t = 0 is the initial state). */
    for (int64_t n = 0; n < N; ++n)
        hist[n] = j->h0 ? j->h0[ch * N + n] : 0.0;
    for (int64_t t = 0; t < len; ++t) {
        double x = dl[t] + bias;
        double dt = j->softplus ? softplus(x) : x;
        double keep = resets(j, b, t) ? 0.0 : 1.0;
        for (int64_t n = 0; n < N; ++n)
            hist[(t + 1) * N + n] = exp(dt * Arow[n]) * keep * hist[t * N + n] + dt * Bb[n * L + t] * u[t];
    }

    for (int64_t n = 0; n < N; ++n)
        g[n] = j->dlast ? j->dlast[ch * N + n] : 0.0;
    for (int64_t t = L - 1; t >= len; --t) {
        j->du[ch * L + t] = 0.0;
        j->ddelta[ch * L + t] = 0.0;
        if (zz) j->dz[ch * L + t] = 0.0;
    }
    for (int64_t t = len - 1; t >= 0; --t) {
        const double *hprev = hist + t * N, *hcur = hist + (t + 1) * N;
        double x = dl[t] + bias;
        double dt = j->softplus ? softplus(x) : x;
        double y0 = Dd * u[t];
        for (int64_t n = 0; n < N; ++n)
            y0 += Cb[n * L + t] * hcur[n];
        double dy0 = dy[t];
        if (zz) {
            double sg = sigmoid(zz[t]);
            dy0 = dy[t] * zz[t] * sg;
            j->dz[ch * L + t] = dy[t] * y0 * sg * (1.0 + zz[t] * (1.0 - sg));
        }
        double du = dy0 * Dd;
        double ddt = 0.0;
        double keep = resets(j, b, t) ? 0.0 : 1.0;      /* h_t = a keep h_{t-1} + ... */
        if (j->Dskip) s->dD[d] += dy0 * u[t];
        for (int64_t n = 0; n < N; ++n) {
            double a = exp(dt * Arow[n]);
            double gh = g[n] + dy0 * Cb[n * L + t];    /* dLoss/dh_t[n]         */
            s->dC[b * N * L + n * L + t] += dy0 * hcur[n];
            s->dB[b * N * L + n * L + t] += gh * dt * u[t];
            du += gh * dt * Bb[n * L + t];
            ddt += gh * (Bb[n * L + t] * u[t] + a * Arow[n] * keep * hprev[n]);
            s->dA[d * N + n] += gh * a * dt * keep * hprev[n];
            g[n] = gh * a * keep;                       /* to h_{t-1}            */
        }
        double dx = j->softplus ? ddt * sigmoid(x) : ddt;
        j->du[ch * L + t] = du;
        j->ddelta[ch * L + t] = dx;
        if (j->bias) s->dbias[d] += dx;
    }
    if (j->dh0)
        for (int64_t n = 0; n < N; ++n)
            j->dh0[ch * N + n] = g[n];                  /* dLoss/dh0             */
}

static void *run_forward(void *arg)
{
    const slice_t *s = (const slice_t *)arg;
    const job_t *j = s->job;
    for (int64_t i = s->first; i < s->last; ++i) {
        int64_t ch = j->rows ? j->rows[i] : i;
        forward_channel(j, ch / j->dim, ch % j->dim);
    }
    return NULL;
}

static void *run_backward(void *arg)
{
    const slice_t *s = (const slice_t *)arg;
    const job_t *j = s->job;
    double *hist = (double *)malloc(sizeof(double) * (size_t)((j->seqlen + 1) * j->dstate));
    if (!hist) return (void *)1;
    for (int64_t i = s->first; i < s->last; ++i)
        backward_channel(s, i / j->dim, i % j->dim, hist);
    free(hist);
    return NULL;
}

static int spawn(job_t *job, int64_t nitems, int nthreads, int backward)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nitems < nthreads) nthreads = (int)(nitems > 0 ? nitems : 1);
    pthread_t tid[256];
    slice_t sl[256];
    const int64_t D = job->dim, N = job->dstate, L = job->seqlen, Bsz = job->batch;
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        memset(&sl[i], 0, sizeof(slice_t));
        sl[i].job = job;
        sl[i].first = nitems * i / nthreads;
        sl[i].last = nitems * (i + 1) / nthreads;
        if (backward) {
            sl[i].dA = (double *)calloc((size_t)(D * N), sizeof(double));
            sl[i].dB = (double *)calloc((size_t)(Bsz * N * L), sizeof(double));
            sl[i].dC = (double *)calloc((size_t)(Bsz * N * L), sizeof(double));
            sl[i].dD = (double *)calloc((size_t)D, sizeof(double));
            sl[i].dbias = (double *)calloc((size_t)D, sizeof(double));
            if (!sl[i].dA || !sl[i].dB || !sl[i].dC || !sl[i].dD || !sl[i].dbias) rc = -2;
        }
    }
    if (rc == 0) {
        for (int i = 0; i < nthreads; ++i)
            pthread_create(&tid[i], NULL, backward ? run_backward : run_forward, &sl[i]);
        for (int i = 0; i < nthreads; ++i) {
            void *ret = NULL;
            pthread_join(tid[i], &ret);
            if (ret) rc = -2;
        }
    }
    if (backward) {
        if (rc == 0) {
            memset(job->dA, 0, sizeof(double) * (size_t)(D * N));
            memset(job->dB, 0, sizeof(double) * (size_t)(Bsz * N * L));
            memset(job->dC, 0, sizeof(double) * (size_t)(Bsz * N * L));
            if (job->dD) memset(job->dD, 0, sizeof(double) * (size_t)D);
            if (job->dbias) memset(job->dbias, 0, sizeof(double) * (size_t)D);
            for (int i = 0; i < nthreads; ++i) {
                for (int64_t k = 0; k < D * N; ++k) job->dA[k] += sl[i].dA[k];
                for (int64_t k = 0; k < Bsz * N * L; ++k) job->dB[k] += sl[i].dB[k];
                for (int64_t k = 0; k < Bsz * N * L; ++k) job->dC[k] += sl[i].dC[k];
                for (int64_t k = 0; k < D; ++k) {
                    if (job->dD) job->dD[k] += sl[i].dD[k];
                    if (job->dbias) job->dbias[k] += sl[i].dbias[k];
                }
            }
        }
        for (int i = 0; i < nthreads; ++i) {
            free(sl[i].dA); free(sl[i].dB); free(sl[i].dC); free(sl[i].dD); free(sl[i].dbias);
        }
    }
    return rc;
}

static int check_shape(int64_t Bsz, int64_t D, int64_t N, int64_t L)
{
    if (Bsz < 1 || D < 1 || N < 1 || N > 64 || L < 1) return -1;
    return 0;
}

/*
 * Forward scan.  All arrays are C-contiguous doubles in the layouts of the
 * problem statement: u, delta, z, y (B,D,L); A (D,N); Bm, Cm (B,N,L);
 * Dskip, bias (D); h0, last_state (B,D,N); seq_idx (B,L).  Dskip, z, bias,
 * lengths, seq_idx, h0, last_state and states may be NULL.  rows (nrows entries of b*D+d) limits
 * the work to those channels; NULL means every channel.  states, when given,
 * receives for every channel K = ceil(L/every) states: entry k is the state
 * after min(k*every, len_b) steps.  Returns 0, or a negative code for a bad
 * shape or an allocation failure.
 */
int sso_fwd(int64_t Bsz, int64_t D, int64_t N, int64_t L, int softplus_flag,
            const double *u, const double *delta, const double *A,
            const double *Bm, const double *Cm, const double *Dskip,
            const double *z, const double *bias, const int64_t *lengths,
            const int64_t *seq_idx, const double *h0, const int64_t *rows, int64_t nrows,
            double *y, double *last_state, double *states, int64_t states_every,
            int nthreads)
{
    if (check_shape(Bsz, D, N, L)) return -1;
    if (!u || !delta || !A || !Bm || !Cm || !y) return -1;
    if (states && states_every < 1) return -1;
    job_t job;
    memset(&job, 0, sizeof(job));
    job.batch = Bsz; job.dim = D; job.dstate = N; job.seqlen = L;
    job.softplus = softplus_flag;
    job.u = u; job.delta = delta; job.A = A; job.Bm = Bm; job.Cm = Cm;
    job.Dskip = Dskip; job.z = z; job.bias = bias; job.lengths = lengths; job.h0 = h0;
    job.seq_idx = seq_idx;
    job.rows = rows; job.nrows = nrows;
    job.y = y; job.last_state = last_state; job.states = states; job.states_every = states_every;
    int64_t nitems = rows ? nrows : Bsz * D;
    return spawn(&job, nitems, nthreads, 0);
}

/*
 * One decode step from a carried state ("mamba-metal" README, O(1) per token
 * via state caching; walkthrough Part IV Stage 7): the forward of a length-1
 * sequence started from state_in.  u_t, delta_t, z_t, y_t are (B,D);
 * B_t, C_t are (B,N); state_in, state_out are (B,D,N) and may be the same
 * array.  Written out on its own rather than by calling sso_fwd.
 */
int sso_step(int64_t Bsz, int64_t D, int64_t N, int softplus_flag,
             const double *u_t, const double *delta_t, const double *A,
             const double *B_t, const double *C_t, const double *Dskip,
             const double *z_t, const double *bias, const double *state_in,
             double *state_out, double *y_t)
{
    if (check_shape(Bsz, D, N, 1)) return -1;
    if (!u_t || !delta_t || !A || !B_t || !C_t || !state_in || !state_out || !y_t) return -1;
    for (int64_t b = 0; b < Bsz; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            const int64_t ch = b * D + d;
            double x = delta_t[ch] + (bias ? bias[d] : 0.0);
            double dt = softplus_flag ? softplus(x) : x;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double a = exp(dt * A[d * N + n]);
                double h = a * state_in[ch * N + n] + dt * B_t[b * N + n] * u_t[ch];
                state_out[ch * N + n] = h;
                acc += C_t[b * N + n] * h;
            }
            if (Dskip) acc += Dskip[d] * u_t[ch];
            if (z_t) acc *= z_t[ch] * sigmoid(z_t[ch]);
            y_t[ch] = acc;
        }
    }
    return 0;
}

/*
 * Backward scan for the loss sum(dy * out) + sum(dlast * h_final).  Inputs
 * as sso_fwd (lengths, seq_idx, h0 and dlast optional); every output is
 * overwritten.  du, ddelta, dz: (B,D,L); dA: (D,N); dB, dC: (B,N,L) summed
 * over d; dD, dbias: (D) summed over b and t; dh0 (B,D,N), optional.  dz
 * must be given iff z is; dD iff Dskip; dbias iff bias.
 */
int sso_bwd(int64_t Bsz, int64_t D, int64_t N, int64_t L, int softplus_flag,
            const double *u, const double *delta, const double *A,
            const double *Bm, const double *Cm, const double *Dskip,
            const double *z, const double *bias, const int64_t *lengths,
            const int64_t *seq_idx, const double *h0, const double *dy, const double *dlast,
            double *du, double *ddelta, double *dz, double *dA,
            double *dB, double *dC, double *dD, double *dbias, double *dh0, int nthreads)
{
    if (check_shape(Bsz, D, N, L)) return -1;
    if (!u || !delta || !A || !Bm || !Cm || !dy || !du || !ddelta || !dA || !dB || !dC) return -1;
    if ((z == NULL) != (dz == NULL) || (Dskip == NULL) != (dD == NULL) || (bias == NULL) != (dbias == NULL))
        return -1;
    job_t job;
    memset(&job, 0, sizeof(job));
    job.batch = Bsz; job.dim = D; job.dstate = N; job.seqlen = L;
    job.softplus = softplus_flag;
    job.u = u; job.delta = delta; job.A = A; job.Bm = Bm; job.Cm = Cm;
    job.Dskip = Dskip; job.z = z; job.bias = bias; job.lengths = lengths; job.h0 = h0; job.dy = dy;
    job.seq_idx = seq_idx; job.dlast = dlast;
    job.du = du; job.ddelta = ddelta; job.dz = dz; job.dA = dA; job.dB = dB; job.dC = dC;
    job.dD = dD; job.dbias = dbias; job.dh0 = dh0;
    return spawn(&job, Bsz * D, nthreads, 1);
}

/*
 * Depthwise causal convolution + SiLU, the step before the scan ("Mamba"
 * walkthrough, Part IV Stage 2: each channel has its own filter of width
 * d_conv; the input is padded on the left only, so position t sees inputs
 * t-W+1 .. t; a SiLU follows).  Plain definition per output:
 *   pre[b,d,t] = bias[d] + sum_{k<W} w[d,k] * x[b,d,t-W+1+k]
 *   out[b,d,t] = silu ? pre * sigmoid(pre) : pre
 * Inputs before t = 0 come from conv_init[b,d,0..W-2] (oldest first) when
 * given, else 0.  With document ids ("niverel-mamba" README, "seq_idx strict
 * reset": the convolution state resets too) an input of another document
 * than step t's counts as 0, and conv_init reaches only the first document.
 * conv_final[b,d,j] = the input at t = L-W+1+j (0 when that is before 0 and
 * no conv_init covers it, or when it belongs to another document than the
 * last step's), the window a decode step continues from.
 * x, out: (B,D,L); w: (D,W); bias: (D) or NULL; seq_idx: (B,L) or NULL;
 * conv_init, conv_final: (B,D,W-1) or NULL.
 */
int sso_conv1d_fwd(int64_t Bsz, int64_t D, int64_t L, int64_t W, int silu,
                   const double *x, const double *w, const double *bias,
                   const int64_t *seq_idx, const double *conv_init,
                   double *out, double *conv_final)
{
    if (Bsz < 1 || D < 1 || L < 1 || W < 1 || W > 16 || !x || !w || !out) return -1;
    for (int64_t b = 0; b < Bsz; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            const int64_t ch = b * D + d;
            const double *xr = x + ch * L;
            /* the input at time s (s may be negative) as seen from step t */
            for (int64_t t = 0; t < L; ++t) {
                double pre = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    int64_t s = t - (W - 1) + k;
                    double v = 0.0;
                    if (s >= 0) {
                        int same = !seq_idx || seq_idx[b * L + s] == seq_idx[b * L + t];
                        v = same ? xr[s] : 0.0;
                    } else if (conv_init) {
                        /* before the row: only the first document sees it */
                        int first = !seq_idx || seq_idx[b * L + t] == seq_idx[b * L];
                        v = first ? conv_init[ch * (W - 1) + (W - 1 + s)] : 0.0;
                    }
                    pre += w[d * W + k] * v;
                }
                out[ch * L + t] = silu ? pre * sigmoid(pre) : pre;
            }
            if (conv_final) {
                for (int64_t j = 0; j < W - 1; ++j) {
                    int64_t s = L - (W - 1) + j;
                    double v = 0.0;
                    if (s >= 0) {
                        int same = !seq_idx || seq_idx[b * L + s] == seq_idx[b * L + L - 1];
                        v = same ? xr[s] : 0.0;
                    } else if (conv_init) {
                        int first = !seq_idx || seq_idx[b * L + L - 1] == seq_idx[b * L];
                        v = first ? conv_init[ch * (W - 1) + (W - 1 + s)] : 0.0;
                    }
                    conv_final[ch * (W - 1) + j] = v;
                }
            }
        }
    }
    return 0;
}

/*
 * One decode step of the convolution: out = silu(bias + sum_{k<W-1} w[k] *
 * window[k] + w[W-1] * x_t); the window (B,D,W-1, oldest first) then drops
 * its oldest input and appends x_t ("mamba-metal" README: the conv1d sliding
 * window is carried across calls).  window_in and window_out may be the same
 * array.  x_t, out_t: (B,D).
 */
int sso_conv1d_step(int64_t Bsz, int64_t D, int64_t W, int silu,
                    const double *x_t, const double *w, const double *bias,
                    const double *window_in, double *window_out, double *out_t)
{
    if (Bsz < 1 || D < 1 || W < 1 || W > 16 || !x_t || !w || !window_in || !window_out || !out_t) return -1;
    for (int64_t b = 0; b < Bsz; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            const int64_t ch = b * D + d;
            double win[16];
            for (int64_t k = 0; k < W - 1; ++k) win[k] = window_in[ch * (W - 1) + k];
            double pre = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < W - 1; ++k) pre += w[d * W + k] * win[k];
            pre += w[d * W + W - 1] * x_t[ch];
            out_t[ch] = silu ? pre * sigmoid(pre) : pre;
            for (int64_t k = 0; k + 1 < W - 1; ++k) window_out[ch * (W - 1) + k] = win[k + 1];
            if (W > 1) window_out[ch * (W - 1) + W - 2] = x_t[ch];
        }
    }
    return 0;
}

/*
 * Mamba-2 structured state-space (SSD) scan, forward ("Mamba" walkthrough,
 * "Deep dive: Mamba-2 and state-space duality": A is a scalar times the
 * identity per head, heads share grouped B and C).  Plain recurrence per
 * (batch b, head h), state H[p][n] (headdim x dstate):
 *   Delta_t  = softplus(dt[b,t,h] + dt_bias[h])   (softplus only if flagged)
 *   a_t      = exp(Delta_t * A[h])
 *   H[p][n]  = a_t H[p][n] + Delta_t x[b,t,h,p] B[b,t,g,n]       g = h / (H/G)
 *   y[b,t,h,p] = sum_n C[b,t,g,n] H[p][n] + D[h] x[b,t,h,p]   (* SiLU(z) if z)
 * starting from h0 (or 0); with document ids the state is zero before every
 * step whose id differs from the previous step's ("niverel-mamba" README,
 * "seq_idx strict reset").  Layouts: x, z, y (B,L,H,P); dt (B,L,H);
 * A, D, dt_bias (H); Bm, Cm (B,L,G,N); h0, final_state (B,H,P,N).
 */
int sso_ssd_fwd(int64_t Bsz, int64_t L, int64_t Hn, int64_t P, int64_t G, int64_t N, int softplus_flag,
                const double *x, const double *dt, const double *A, const double *Bm, const double *Cm,
                const double *Dskip, const double *z, const double *dt_bias, const int64_t *seq_idx,
                const double *h0, double *y, double *final_state)
{
    if (Bsz < 1 || L < 1 || Hn < 1 || P < 1 || G < 1 || N < 1 || Hn % G != 0) return -1;
    if (!x || !dt || !A || !Bm || !Cm || !y) return -1;
    double *Hs = (double *)malloc(sizeof(double) * (size_t)(P * N));
    if (!Hs) return -2;
    const int64_t hpg = Hn / G;
    for (int64_t b = 0; b < Bsz; ++b) {
        for (int64_t h = 0; h < Hn; ++h) {
            const int64_t g = h / hpg;
            for (int64_t i = 0; i < P * N; ++i)
                Hs[i] = h0 ? h0[(b * Hn + h) * P * N + i] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                if (seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1])
                    for (int64_t i = 0; i < P * N; ++i) Hs[i] = 0.0;      /* a new document */
                double xd = dt[(b * L + t) * Hn + h] + (dt_bias ? dt_bias[h] : 0.0);
                double delta = softplus_flag ? softplus(xd) : xd;
                double a = exp(delta * A[h]);
                const double *Bt = Bm + ((b * L + t) * G + g) * N;
                const double *Ct = Cm + ((b * L + t) * G + g) * N;
                const double *xt = x + ((b * L + t) * Hn + h) * P;
                double *yt = y + ((b * L + t) * Hn + h) * P;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        Hs[p * N + n] = a * Hs[p * N + n] + delta * xt[p] * Bt[n];
                        acc += Ct[n] * Hs[p * N + n];
                    }
                    if (Dskip) acc += Dskip[h] * xt[p];
                    if (z) {
                        double zz = z[((b * L + t) * Hn + h) * P + p];
                        acc *= zz * sigmoid(zz);
                    }
                    yt[p] = acc;
                }
            }
            if (final_state)
                for (int64_t i = 0; i < P * N; ++i) final_state[(b * Hn + h) * P * N + i] = Hs[i];
        }
    }
    free(Hs);
    return 0;
}
