/* Test infrastructure: the oracle's fixed-point selective scan in plain C.
 *
 * The same definition as ssm_scan_pot in oracle/scan.py (FastMamba paper,
 * Fig. 2 SSM block; review page "What carries the argument": power-of-two
 * scaling makes every rescaling a shift), written out again so that whole
 * layers at their full sizes finish in seconds: per (batch, head, p, n), t
 * ascending, in exact 64-bit integers,
 *     u   = dt * x_q
 *     h_t = sat32(floor((dA * h_{t-1} + 2^8 * u * B_q + 2^15) / 2^16))
 *     y   = sat32(rshr(sum_n C_q * h_t, p_B + p_C) + rshr(D_q16 * x_q, 8))
 * with rshr(v, s) = floor(v / 2^s + 1/2) for s > 0, v for s = 0 and the exact
 * product v * 2^-s (clamped to +-2^62) for s < 0.  Magnitudes: |dA * h| <
 * 2^47, |2^8 u B| < 2^54, |sum C h| < 2^45: no intermediate leaves int64.
 *
 * Only tests load this library; nothing of the device library uses it.  It
 * takes a range [bh0, bh1) of (batch, head) pairs so that callers can run
 * ranges on several threads. */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LIM62 ((int64_t)1 << 62)

static int64_t sat32(int64_t v) {
    if (v < -((int64_t)1 << 31)) return -((int64_t)1 << 31);
    if (v > ((int64_t)1 << 31) - 1) return ((int64_t)1 << 31) - 1;
    return v;
}

static int64_t rshr(int64_t v, int s) {
    if (s >= 63) return 0;
    if (s >= 1) {
        const int64_t q = (v + ((int64_t)1 << (s - 1)));
        return q >= 0 ? q >> s : -((-q + ((int64_t)1 << s) - 1) >> s);  /* floor */
    }
    if (s == 0) return v;
    const int k = -s;
    if (k >= 62) return v > 0 ? LIM62 : (v < 0 ? -LIM62 : 0);
    const int64_t lim = LIM62 >> k;
    if (v >= lim) return LIM62;
    if (v <= -lim) return -LIM62;
    return v * ((int64_t)1 << k);
}

/* x [Bsz, L, H, P] int8; bm, cm [Bsz, L, N] int8; dt, da [Bsz, L, H] int64;
 * d_q16 [H] int64; state_in [Bsz, H, P, N] int64 or NULL (zeros);
 * y [Bsz, L, H, P] int64 and state_out [Bsz, H, P, N] int64 written for the
 * (b, h) pairs bh in [bh0, bh1), bh = b * H + h.  Returns 0, or -1 when a
 * scratch allocation fails. */
int oracle_scan_range(const int8_t* x, const int8_t* bm, const int8_t* cm, const int64_t* dt,
                      const int64_t* da, const int64_t* d_q16, int p_B, int p_C, int64_t Bsz,
                      int64_t L, int64_t H, int64_t P, int64_t N, const int64_t* state_in,
                      int64_t* y, int64_t* state_out, int64_t bh0, int64_t bh1) {
    (void)Bsz;
    int64_t* hs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(P * N));
    if (!hs) return -1;
    const int ky = p_B + p_C;
    for (int64_t bh = bh0; bh < bh1; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        if (state_in)
            memcpy(hs, state_in + bh * P * N, sizeof(int64_t) * (size_t)(P * N));
        else
            memset(hs, 0, sizeof(int64_t) * (size_t)(P * N));
        for (int64_t t = 0; t < L; ++t) {
            const int64_t bt = b * L + t;
            const int64_t dtv = dt[bt * H + h], dav = da[bt * H + h];
            const int8_t* bt_b = bm + bt * N;
            const int8_t* bt_c = cm + bt * N;
            for (int64_t p = 0; p < P; ++p) {
                const int64_t xv = x[(bt * H + h) * P + p];
                const int64_t u = dtv * xv;
                int64_t* hr = hs + p * N;
                int64_t acc = 0;
                for (int64_t n = 0; n < N; ++n) {
                    const int64_t inc = (u * (int64_t)bt_b[n]) * 256;
                    const int64_t num = dav * hr[n] + inc + ((int64_t)1 << 15);
                    /* floor division by 2^16 */
                    const int64_t q = num >= 0 ? num >> 16 : -((-num + 65535) >> 16);
                    hr[n] = sat32(q);
                    acc += (int64_t)bt_c[n] * hr[n];
                }
                y[(bt * H + h) * P + p] = sat32(rshr(acc, ky) + rshr(d_q16[h] * xv, 8));
            }
        }
        memcpy(state_out + bh * P * N, hs, sizeof(int64_t) * (size_t)(P * N));
    }
    free(hs);
    return 0;
}
