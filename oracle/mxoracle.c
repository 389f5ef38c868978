/*
 * mxoracle.c -- CPU oracle for MXFP4 attention with UOS and PNQ.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent, slow, obviously
 * correct model that the GPU path is checked against.  Only the test suite,
 * the package smoke check and the CPU-baseline leg of the benchmark may load
 * it.  It shares no code, header, table or constant generator with the HIP
 * library, and the HIP library never calls it.
 *
 * Source of the method: "MXAttention: Data-Free Optimal Scaling and
 * Pre-Normalization Quantization for MXFP4 Attention" (arXiv 2607.24377),
 * abstract.  The abstract names the pieces and fixes one constant:
 *   - MXFP4 elements share a power-of-two scale per block;
 *   - OCP MXFP4 is the baseline quantizer;
 *   - Universal Optimal Scaling (UOS) picks the block scale from a fixed,
 *     data-free boundary Qmax = 7.25;
 *   - Pre-Normalization Quantization (PNQ) quantizes the unnormalized
 *     exponentials of the online softmax before the row sum, so the row sum and
 *     the P.V product see the same quantized values.
 * Everything the abstract leaves open (block size 32, E2M1 elements, E8M0
 * scales, round-to-nearest-even, blocking axes, the running-max schedule,
 * the meaning of "PNQ off") is a stated reading; each function says which.
 *
 * Precision: values, sums and the softmax recurrence are fp64.  Where the
 * GPU kernel takes an integer decision from an fp32 value (the code of an
 * exponential, a block scale), the oracle rounds that value to fp32 first,
 * so both sides decide from the same precision.
 *
 * Pins: every function here is checked by the host tests against facts that
 * do not come from this file (hand-worked blocks, interval invariants, the
 * brute-force MSE optimum of the scale boundary, textbook attention, closed
 * forms of the recurrence, the normalization invariant of PNQ).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MODE_OCP 0
#define ORC_MODE_UOS 1
#define ORC_MODE_NONE 2 /* identity quantizer: used only to reduce the
                           oracle to textbook attention in the pins */

/* The eight E2M1 magnitudes, indexed by the 3-bit code (exponent bits 2:1,
 * mantissa bit 0).  OCP E2M1 value set; bit 3 of a code is the sign. */
static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* UOS boundary from the abstract. */
static const double kUosQmax = 7.25;

/* OCP: the largest element exponent of E2M1 (6 = 1.5 * 2^2). */
static const int kE2M1Emax = 2;

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to bf16, round-to-nearest-even (the oracle's bf16 copy of
 * the output).  The bf16 grid spacing at |x| is 2^(E-7) with E the binary
 * exponent of |x| (E >= -126, below that the spacing stays 2^-133);
 * x / spacing is exact and nearbyint() rounds it half-to-even. */
uint16_t orc_double_to_bf16(double x)
{
    if (x == 0.0)
        return signbit(x) ? 0x8000u : 0x0000u;
    int fe;
    frexp(fabs(x), &fe);
    int E = fe - 1;
    if (E < -126)
        E = -126;
    double ulp = ldexp(1.0, E - 7);
    double r = nearbyint(x / ulp) * ulp;
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* E2M1 encode of y, where y is the element already divided by its block
 * scale.  Reading (OCP E2M1, round-to-nearest-even, saturating): the code is
 * the nearest of the eight magnitudes; on a tie the even code wins; anything
 * beyond 6 lands on 6.  The sign bit is the sign bit of y, so a negative value
 * that rounds to zero keeps its sign (code 0x8). */
int orc_e2m1_encode(double y)
{
    int neg = signbit(y) ? 1 : 0;
    double a = fabs(y);
    if (a > 6.0) /* saturate: 6 is the nearest magnitude to anything above it */
        a = 6.0;
    int best = 0;
    double bestd = fabs(a - kE2M1Mag[0]);
    for (int c = 1; c < 8; ++c) {
        double dist = fabs(a - kE2M1Mag[c]);
        if (dist < bestd || (dist == bestd && (c & 1) == 0)) {
            best = c;
            bestd = dist;
        }
    }
    return best | (neg << 3);
}

/* Value of a 4-bit code under block exponent e. */
double orc_e2m1_value(int code, int e)
{
    double m = kE2M1Mag[code & 7];
    if (code & 8)
        m = -m;
    return ldexp(m, e);
}

/* Block exponent for a block whose largest magnitude is amax.
 *   OCP (baseline named in the abstract; reading = the OCP MX rule):
 *       e = floor(log2 amax) - 2, so amax / 2^e lies in [4, 8).
 *   UOS (abstract: boundary Qmax = 7.25; reading = the smallest power-of-two
 *       scale that keeps amax / scale <= 7.25):
 *       e = the least integer with amax <= 7.25 * 2^e, so amax / 2^e lies in
 *       (3.625, 7.25]; values between 6 and 7.25 then saturate to 6.
 * A zero block takes the smallest E8M0 scale.  e is clamped to the E8M0
 * range [-127, 127] (byte 255 is NaN in E8M0 and is never produced). */
int orc_block_exponent(double amax, int mode)
{
    int e;
    if (!(amax > 0.0))
        return -127;
    int fe;
    frexp(amax, &fe); /* amax = f * 2^fe with f in [0.5, 1) */
    int floor_log2 = fe - 1;
    if (mode == ORC_MODE_OCP) {
        e = floor_log2 - kE2M1Emax;
    } else {
        e = floor_log2 - 4; /* 7.25 * 2^e < amax here */
        while (amax > ldexp(kUosQmax, e))
            ++e;
    }
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* Quantize one vector of len values (x[i * stride]) in blocks of 32 along the
 * vector.  The last block is zero-padded.  codes: nb*16 bytes, element 2i of a
 * block in bits 3:0 of byte i, element 2i+1 in bits 7:4.  scales: nb E8M0
 * bytes (e + 127). */
static void quant_vec(const double *x, int64_t len, int64_t stride, int mode, uint8_t *codes,
                      uint8_t *scales)
{
    int64_t nb = (len + 31) / 32;
    for (int64_t b = 0; b < nb; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            int64_t idx = b * 32 + i;
            if (idx < len) {
                double a = fabs(x[idx * stride]);
                if (a > amax)
                    amax = a;
            }
        }
        int e = orc_block_exponent(amax, mode);
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 16; ++i) {
            int code[2];
            for (int h = 0; h < 2; ++h) {
                int64_t idx = b * 32 + 2 * i + h;
                double v = idx < len ? x[idx * stride] : 0.0;
                code[h] = orc_e2m1_encode(ldexp(v, -e));
            }
            codes[b * 16 + i] = (uint8_t)(code[0] | (code[1] << 4));
        }
    }
}

static int check_finite(const double *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i]))
            return 0;
    return 1;
}

/* Quantize bf16 x viewed as [batch][rows][cols] in blocks of 32 along axis
 * (1: along cols, the contiguous axis; 0: along rows).
 *   axis 1: codes [batch][rows][nb*16], scales [batch][rows][nb], nb = ceil(cols/32)
 *   axis 0: codes [batch][cols][nb*16], scales [batch][cols][nb], nb = ceil(rows/32)
 * Returns 0, or -1 on a bad argument or a non-finite input. */
int orc_quantize_bf16(const uint16_t *x, int64_t batch, int64_t rows, int64_t cols, int axis,
                      int mode, uint8_t *codes, uint8_t *scales)
{
    if (batch < 0 || rows < 0 || cols < 0 || (axis != 0 && axis != 1) ||
        (mode != ORC_MODE_OCP && mode != ORC_MODE_UOS))
        return -1;
    int64_t per = rows * cols;
    double *buf = (double *)malloc((size_t)(per > 0 ? per : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t bi = 0; bi < batch; ++bi) {
        for (int64_t i = 0; i < per; ++i)
            buf[i] = orc_bf16_to_double(x[bi * per + i]);
        if (!check_finite(buf, per)) {
            free(buf);
            return -1;
        }
        if (axis == 1) {
            int64_t nb = (cols + 31) / 32;
            for (int64_t r = 0; r < rows; ++r)
                quant_vec(buf + r * cols, cols, 1, mode, codes + (bi * rows + r) * nb * 16,
                          scales + (bi * rows + r) * nb);
        } else {
            int64_t nb = (rows + 31) / 32;
            for (int64_t c = 0; c < cols; ++c)
                quant_vec(buf + c, rows, cols, mode, codes + (bi * cols + c) * nb * 16,
                          scales + (bi * cols + c) * nb);
        }
    }
    free(buf);
    return 0;
}

/* Quantize an fp64 vector (any values; used by the pins on fp32-rounded
 * exponentials and on random blocks). */
int orc_quantize_f64(const double *x, int64_t len, int mode, uint8_t *codes, uint8_t *scales)
{
    if (len < 0 || (mode != ORC_MODE_OCP && mode != ORC_MODE_UOS) || !check_finite(x, len))
        return -1;
    quant_vec(x, len, 1, mode, codes, scales);
    return 0;
}

/* Dequantize a canonical code/scale pair of arrays for nvec vectors of
 * length L (padding dropped): out[v * L + i]. */
void orc_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t nvec, int64_t L, double *out)
{
    int64_t nb = (L + 31) / 32;
    for (int64_t vI = 0; vI < nvec; ++vI)
        for (int64_t i = 0; i < L; ++i) {
            int64_t b = i / 32, w = i % 32;
            uint8_t byte = codes[(vI * nb + b) * 16 + w / 2];
            int code = (w & 1) ? (byte >> 4) : (byte & 15);
            out[vI * L + i] = orc_e2m1_value(code, (int)scales[vI * nb + b] - 127);
        }
}

/* Sum of squared errors of one block quantized with a given exponent e
 * (any e, no rule).  Used by the brute-force search over scales. */
double orc_block_sse(const double *x, int64_t n, int e)
{
    double sse = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double q = orc_e2m1_value(orc_e2m1_encode(ldexp(x[i], -e)), e);
        double d = x[i] - q;
        sse += d * d;
    }
    return sse;
}

/* Batch form: nblk blocks of n values; for each block, the SSE at each of
 * ne exponents e0 + j (j < ne), into sse[blk * ne + j]. */
void orc_block_sse_batch(const double *x, int64_t nblk, int64_t n, int e0, int ne, double *sse)
{
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b)
        for (int j = 0; j < ne; ++j)
            sse[b * ne + j] = orc_block_sse(x + b * n, n, e0 + j);
}

/* Relative distance of y (>= 0) to the nearest decision point of the E2M1
 * encoder (the midpoints between neighbouring magnitudes). */
static double e2m1_tie_distance(double y)
{
    static const double thr[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    double best = INFINITY;
    for (int i = 0; i < 7; ++i) {
        double r = fabs(y - thr[i]) / thr[i];
        if (r < best)
            best = r;
    }
    return best;
}

/* Relative distance of amax to the nearest point where the block exponent
 * changes under the given rule. */
static double scale_boundary_distance(double amax, int mode)
{
    if (!(amax > 0.0))
        return INFINITY;
    int fe;
    double f = frexp(amax, &fe); /* f in [0.5, 1) */
    double m = 2.0 * f;          /* mantissa in [1, 2) */
    double best = fmin(fabs(m - 1.0), fabs(2.0 - m) / 2.0);
    if (mode == ORC_MODE_UOS) {
        double r = fabs(m - 1.8125) / 1.8125;
        if (r < best)
            best = r;
    }
    return best;
}

/* Quantize one P block held in fp32-rounded doubles p[0..n) (n <= 32, the
 * rest of the 32-key block is padding) into p_hat.  Returns 1 when one of the
 * block's decisions (its scale, or an element's code) lies so close to a
 * boundary that the fp32 definition of p does not settle it.
 *
 * The exponential is defined from fp32 scores t (t = fp32(s * scale)) and the
 * running max m, so p itself is only fixed to about 2^-24 (|t| + |m|)
 * relative: any fp32 evaluation order moves it by that much.  A decision is
 * flagged when it lies within eps = 2^-22 (4 + |t| + |m|) of a tie (relative),
 * which covers the roundings of t, m, the scale product and the exponential.
 * Blocks whose largest exponential is below 2^-60 are never flagged: their
 * weights cannot reach any output at the acceptance tolerance.  An amax of
 * exactly 1 (the block holding the running max) is exact on every side. */
/* Largest change of the quantized value of p (block exponent e, quantized
 * value ph) when p moves by a relative eps either way: the encoder is
 * monotone, so the two ends of the interval bound every outcome. */
static double alt_change(double p, double eps, int e, double ph)
{
    double lo = orc_e2m1_value(orc_e2m1_encode(ldexp(p * (1.0 - eps), -e)), e);
    double hi = orc_e2m1_value(orc_e2m1_encode(ldexp(p * (1.0 + eps), -e)), e);
    return fmax(fabs(lo - ph), fabs(hi - ph));
}

/* dp_hat (may be NULL): for each element, the largest change of its quantized
 * value that a flagged decision allows, i.e. the other side of every tie
 * within eps: its own code, and the block exponent the other side of a scale
 * boundary would take (0 where nothing is that close). */
static int quant_p_block(const double *p, const double *t, double m, int n, int mode,
                         double *p_hat, double *dp_hat)
{
    double amax = 0.0, tmax = -INFINITY;
    for (int i = 0; i < n; ++i) {
        if (p[i] > amax)
            amax = p[i];
        if (t[i] > tmax)
            tmax = t[i];
    }
    int e = orc_block_exponent(amax, mode);
    int near = 0;
    const int relevant = amax >= 0x1p-60;
    const double eps_b = 0x1p-22 * (4.0 + fabs(tmax) + fabs(m));
    if (relevant && amax != 1.0 && scale_boundary_distance(amax, mode) < eps_b)
        near = 1;
    for (int i = 0; i < n; ++i) {
        double y = ldexp(p[i], -e);
        p_hat[i] = orc_e2m1_value(orc_e2m1_encode(y), e);
        if (relevant && y > 0.0 && e2m1_tie_distance(y) < 0x1p-22 * (4.0 + fabs(t[i]) + fabs(m)))
            near = 1;
    }
    if (dp_hat) {
        /* block exponents the other side of a nearby scale boundary */
        int alt[2], nalt = 0;
        if (amax > 0.0 && amax != 1.0) {
            int lo = orc_block_exponent(amax * (1.0 - eps_b), mode);
            int hi = orc_block_exponent(amax * (1.0 + eps_b), mode);
            if (lo != e)
                alt[nalt++] = lo;
            if (hi != e)
                alt[nalt++] = hi;
        }
        for (int i = 0; i < n; ++i) {
            const double eps = 0x1p-22 * (4.0 + fabs(t[i]) + fabs(m));
            double dmax = alt_change(p[i], eps, e, p_hat[i]);
            for (int a = 0; a < nalt; ++a)
                dmax = fmax(dmax, alt_change(p[i], eps, alt[a], p_hat[i]));
            dp_hat[i] = dmax;
        }
    }
    return near;
}

/*
 * Non-causal scaled-dot-product attention for selected query rows, with
 * MXFP4 quantization of Q, K, V and of the softmax exponentials.
 *
 * q, k, v: bf16 [BH][N][d] (row-major).  rows[i] in [0, BH*N) picks the
 * query row (head = rows[i] / N).  Outputs per requested row:
 *   out[i*d + c]   O = (sum_k w_k v_k) in fp64 (before bf16 rounding),
 *   lsum[i]        the final row sum l (may be NULL),
 *   flags[i]       bit 0: a P decision lay within the fp32 resolution of p
 *                  of a tie (see quant_p_block; may be NULL),
 *   weights[i*N+k] explicit weights w_k with O = sum_k w_k * deq(v_k)
 *                  (may be NULL; costs O(N^2 / Bc) per row),
 *   budget[i*d+c]  a bound on how far O may move when every flagged
 *                  decision of the row goes the other way (may be NULL):
 *                  with D_k the largest change of the k-th quantized
 *                  exponential (quant_p_block), carried through the same
 *                  rescales as O and l, |dO_c| <= (sum_k D_k |v_kc| +
 *                  |O_c| sum_k D_k) / (l - sum_k D_k), the l terms only
 *                  under PNQ (without it l does not use the codes).  Zero
 *                  for rows with no flagged decision.
 *
 * Readings of the abstract (its only description of the loop is "softmax
 * loop" plus the PNQ sentence):
 *   - Q and K are blocked along d; V along N per channel (MX blocks must lie
 *     along each contraction's reduction axis); a partial last V block is
 *     zero-padded.
 *   - s_j = Q_q . K_q,j exactly (fp64), rounded to fp32; t_j = fp32(s_j * scale).
 *   - The running max is updated once per key tile of Bc keys, tiles in
 *     ascending key order (flash-attention style); Bc is a multiple of 32.
 *   - p_j = fp32(exp(t_j - m')) with m' the running max after the tile; p is
 *     quantized in 32-key blocks aligned to the absolute key index, with the
 *     same scale rule (mode) as Q, K and V.
 *   - PNQ on: the row sum adds the quantized p; PNQ off: it adds the fp32 p.
 *     In both cases the P.V product uses the quantized p.
 *   - mode ORC_MODE_NONE skips every quantization (pins only).
 * Returns 0, or -1 on a bad argument / non-finite input.
 */
int orc_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t BH, int64_t N,
                  int64_t d, int mode, int pnq, int64_t Bc, double softmax_scale, const int64_t *rows,
                  int64_t nrows, double *out, double *lsum, int *flags, double *weights, double *budget)
{
    if (BH < 1 || N < 1 || d < 1 || d % 32 != 0 || Bc < 32 || Bc % 32 != 0 || nrows < 0 ||
        (mode != ORC_MODE_OCP && mode != ORC_MODE_UOS && mode != ORC_MODE_NONE))
        return -1;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= BH * N)
            return -1;
    const float scale32 = (float)softmax_scale;
    const int64_t nbd = d / 32;
    const int64_t nbn = (N + 31) / 32;
    int status = 0;

    double *kd = (double *)malloc((size_t)(N * d) * sizeof(double));
    double *vd = (double *)malloc((size_t)(N * d) * sizeof(double));
    double *tmp = (double *)malloc((size_t)(N * d) * sizeof(double));
    uint8_t *codes = (uint8_t *)malloc((size_t)(nbn * 16 * d + N * nbd * 16));
    uint8_t *scl = (uint8_t *)malloc((size_t)(nbn * d + N * nbd));
    if (!kd || !vd || !tmp || !codes || !scl) {
        free(kd); free(vd); free(tmp); free(codes); free(scl);
        return -1;
    }

    for (int64_t h = 0; h < BH && status == 0; ++h) {
        int any = 0;
        for (int64_t i = 0; i < nrows; ++i)
            if (rows[i] / N == h)
                any = 1;
        if (!any)
            continue;
        /* K of this head: blocks along d; V: blocks along N per channel. */
        const uint16_t *kh = k + h * N * d, *vh = v + h * N * d;
        for (int64_t i = 0; i < N * d; ++i)
            tmp[i] = orc_bf16_to_double(kh[i]);
        if (!check_finite(tmp, N * d)) { status = -1; break; }
        if (mode == ORC_MODE_NONE) {
            memcpy(kd, tmp, (size_t)(N * d) * sizeof(double));
        } else {
            for (int64_t j = 0; j < N; ++j)
                quant_vec(tmp + j * d, d, 1, mode, codes + j * nbd * 16, scl + j * nbd);
            orc_dequantize(codes, scl, N, d, kd);
        }
        for (int64_t i = 0; i < N * d; ++i)
            tmp[i] = orc_bf16_to_double(vh[i]);
        if (!check_finite(tmp, N * d)) { status = -1; break; }
        if (mode == ORC_MODE_NONE) {
            memcpy(vd, tmp, (size_t)(N * d) * sizeof(double));
        } else {
            /* channel c: N values with stride d -> codes [d][nbn*16] */
            for (int64_t c = 0; c < d; ++c)
                quant_vec(tmp + c, N, d, mode, codes + c * nbn * 16, scl + c * nbn);
            double *chan = (double *)malloc((size_t)N * sizeof(double));
            if (!chan) { status = -1; break; }
            for (int64_t c = 0; c < d; ++c) {
                orc_dequantize(codes + c * nbn * 16, scl + c * nbn, 1, N, chan);
                for (int64_t j = 0; j < N; ++j)
                    vd[j * d + c] = chan[j];
            }
            free(chan);
        }

#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t ri = 0; ri < nrows; ++ri) {
            if (rows[ri] / N != h)
                continue;
            int64_t row = rows[ri];
            double *qd = (double *)malloc((size_t)d * sizeof(double));
            double *t = (double *)malloc((size_t)N * sizeof(double));
            double *p = (double *)malloc((size_t)N * sizeof(double));
            double *ph = (double *)malloc((size_t)N * sizeof(double));
            double *O = (double *)calloc((size_t)d, sizeof(double));
            double *dph = budget ? (double *)malloc((size_t)N * sizeof(double)) : NULL;
            double *Bv = budget ? (double *)calloc((size_t)d, sizeof(double)) : NULL;
            double Dl = 0.0;
            uint8_t qc[16 * 8], qs[8];
            double *w = weights ? weights + ri * N : NULL;
            int near = 0;
            /* quantized query row, blocks along d */
            for (int64_t c = 0; c < d; ++c)
                qd[c] = orc_bf16_to_double(q[row * d + c]);
            if (mode != ORC_MODE_NONE) {
                uint8_t *qcb = (d / 32 <= 8) ? qc : (uint8_t *)malloc((size_t)(d / 32) * 16);
                uint8_t *qsb = (d / 32 <= 8) ? qs : (uint8_t *)malloc((size_t)(d / 32));
                quant_vec(qd, d, 1, mode, qcb, qsb);
                orc_dequantize(qcb, qsb, 1, d, qd);
                if (qcb != qc) { free(qcb); free(qsb); }
            }
            /* scores: exact dot of dequantized values, then the two fp32 roundings */
            for (int64_t j = 0; j < N; ++j) {
                double s = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    s += qd[c] * kd[j * d + c];
                float s32 = (float)s;
                t[j] = (double)(float)((double)s32 * (double)scale32);
            }
            double m = -INFINITY, l = 0.0;
            if (w)
                for (int64_t j = 0; j < N; ++j)
                    w[j] = 0.0;
            for (int64_t t0 = 0; t0 < N; t0 += Bc) {
                int64_t t1 = t0 + Bc < N ? t0 + Bc : N;
                double mt = -INFINITY;
                for (int64_t j = t0; j < t1; ++j)
                    if (t[j] > mt)
                        mt = t[j];
                double mnew = m > mt ? m : mt;
                double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
                for (int64_t j = t0; j < t1; ++j)
                    p[j] = (double)(float)exp(t[j] - mnew);
                if (mode == ORC_MODE_NONE) {
                    for (int64_t j = t0; j < t1; ++j) {
                        ph[j] = p[j];
                        if (dph)
                            dph[j] = 0.0;
                    }
                } else {
                    for (int64_t b0 = t0; b0 < t1; b0 += 32) {
                        int n = (int)(t1 - b0 < 32 ? t1 - b0 : 32);
                        near |= quant_p_block(p + b0, t + b0, mnew, n, mode, ph + b0, dph ? dph + b0 : NULL);
                    }
                }
                if (dph) {
                    double ds = 0.0;
                    for (int64_t j = t0; j < t1; ++j)
                        ds += dph[j];
                    Dl = alpha * Dl + (pnq ? ds : 0.0);
                    for (int64_t c = 0; c < d; ++c) {
                        double acc = 0.0;
                        for (int64_t j = t0; j < t1; ++j)
                            acc += dph[j] * fabs(vd[j * d + c]);
                        Bv[c] = alpha * Bv[c] + acc;
                    }
                }
                double rs = 0.0;
                for (int64_t j = t0; j < t1; ++j)
                    rs += pnq ? ph[j] : p[j];
                l = alpha * l + rs;
                for (int64_t c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int64_t j = t0; j < t1; ++j)
                        acc += ph[j] * vd[j * d + c];
                    O[c] = alpha * O[c] + acc;
                }
                if (w) {
                    for (int64_t j = 0; j < t0; ++j)
                        w[j] *= alpha;
                    for (int64_t j = t0; j < t1; ++j)
                        w[j] = ph[j];
                }
                m = mnew;
            }
            for (int64_t c = 0; c < d; ++c)
                out[ri * d + c] = O[c] / l;
            if (budget)
                for (int64_t c = 0; c < d; ++c)
                    budget[ri * d + c] = (Bv[c] == 0.0 && Dl == 0.0) ? 0.0
                                         : (l > Dl ? (Bv[c] + fabs(O[c] / l) * Dl) / (l - Dl) : INFINITY);
            if (w)
                for (int64_t j = 0; j < N; ++j)
                    w[j] /= l;
            if (lsum)
                lsum[ri] = l;
            if (flags)
                flags[ri] = near;
            free(qd); free(t); free(p); free(ph); free(O); free(dph); free(Bv);
        }
    }
    free(kd); free(vd); free(tmp); free(codes); free(scl);
    return status;
}

/* Write a reference-format dump ("MXQ1"): a 256-byte header of ASCII JSON
 * padded with spaces and ending in '\n', then the code bytes, then the scale
 * bytes, both in the canonical layout.  Returns 0 or -1. */
int orc_dump(const char *path, const uint8_t *codes, const uint8_t *scales, int64_t batch,
             int64_t nvec, int64_t L, int axis, int mode)
{
    if (!path || batch < 0 || nvec < 0 || L < 0 || (axis != 0 && axis != 1) ||
        (mode != ORC_MODE_OCP && mode != ORC_MODE_UOS))
        return -1;
    int64_t nb = (L + 31) / 32;
    int64_t ncode = batch * nvec * nb * 16, nscale = batch * nvec * nb;
    char hdr[256];
    int len = snprintf(hdr, sizeof hdr,
                       "{\"magic\":\"MXQ1\",\"version\":1,\"mode\":\"%s\",\"axis\":%d,\"batch\":%lld,"
                       "\"nvec\":%lld,\"L\":%lld,\"block\":32,\"elem\":\"e2m1\",\"scale\":\"e8m0\","
                       "\"nibble\":\"lo-first\"}",
                       mode == ORC_MODE_OCP ? "ocp" : "uos", axis, (long long)batch,
                       (long long)nvec, (long long)L);
    if (len < 0 || len > 254)
        return -1;
    for (int i = len; i < 255; ++i)
        hdr[i] = ' ';
    hdr[255] = '\n';
    FILE *f = fopen(path, "wb");
    if (!f)
        return -1;
    int ok = fwrite(hdr, 1, 256, f) == 256 &&
             fwrite(codes, 1, (size_t)ncode, f) == (size_t)ncode &&
             fwrite(scales, 1, (size_t)nscale, f) == (size_t)nscale;
    ok = (fclose(f) == 0) && ok;
    return ok ? 0 : -1;
}

/* Array form of orc_double_to_bf16. */
void orc_double_to_bf16_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_double_to_bf16(x[i]);
}

/* Array form of orc_e2m1_encode. */
void orc_e2m1_encode_array(const double *y, int64_t n, uint8_t *codes)
{
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (uint8_t)orc_e2m1_encode(y[i]);
}

/* Array form of orc_block_exponent. */
void orc_block_exponent_array(const double *amax, int64_t n, int mode, int32_t *e)
{
    for (int64_t i = 0; i < n; ++i)
        e[i] = orc_block_exponent(amax[i], mode);
}

/* Number of OpenMP threads the row loop uses. */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of OpenMP threads later calls use (timing only). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
