/* Float64 CPU oracle of the RWKV-7 WKV recurrence, in plain C.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg load this library. The product path never
 * calls it, and it shares no code with the HIP kernels or their host
 * library.
 *
 * It computes exactly what oracle/wkv7_oracle.py computes (the same per-
 * element definition, token by token), written as plain loops so that the
 * full-size workloads can be checked element by element in seconds rather
 * than minutes. Page "RWKV-X Architecture", section "WKV-7 Kernel
 * (Generalized Delta Rule)": per head a [head_size, head_size] state is
 * updated once per timestep by a decay, a delta-rule term and a key-value
 * outer product, and the output is read from the state. Reading taken (the
 * page's four pseudocode lines do not type-check as printed): the product
 * form of the generalized delta rule
 *
 *     S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,   o_t = S_t r_t,
 *
 * with S[i][j], i the value index (row) and j the key index (column):
 *
 *     sa[i]     = sum_j S_{t-1}[i][j] a_t[j]       (state before the decay)
 *     S_t[i][j] = S_{t-1}[i][j] w_t[j] + sa[i] b_t[j] + v_t[i] k_t[j]
 *     o_t[i]    = sum_j S_t[i][j] r_t[j]           (the updated state)
 *
 * Nothing is clamped. Inputs are read as float64, float32 or bfloat16 bit
 * patterns and widened exactly (a bfloat16 value is the upper half of the
 * float32 with the same bits), so the oracle consumes the very values the
 * device receives. Build without contraction into fused multiply-adds and
 * without reassociation (-ffp-contract=off, no -ffast-math).
 */
#include <stdint.h>
#include <string.h>

enum { REF_F64 = 0, REF_F32 = 1, REF_BF16 = 2 };

static double widen(const void *p, int dtype, int64_t idx)
{
    if (dtype == REF_F64)
        return ((const double *)p)[idx];
    if (dtype == REF_F32)
        return (double)((const float *)p)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The recurrence over T timesteps for heads [h0, h1) of a block of n_heads
 * independent heads.
 *
 * in[0..5] = r, w, k, v, a, b, each [T][n_heads][N] in `dtype`, row-major
 * (token t, head h, channel c at (t * n_heads + h) * N + c).
 * S: [n_heads][N][N] float64, the start states on entry and the final states
 * on return (only heads h0..h1-1 are touched).
 * o: [T][n_heads][N] float64 outputs (only heads h0..h1-1 are written).
 * A decode batch of B slots with H heads each is T = 1, n_heads = B * H.
 * Returns 0, or -1 for an invalid argument (nothing is written then).
 */
int wkv7_ref_run(int64_t T, int64_t n_heads, int64_t N, int dtype,
                 const void *const in[6], double *S, double *o,
                 int64_t h0, int64_t h1)
{
    if (T < 0 || n_heads < 0 || N <= 0 || N > 1024 || h0 < 0 || h1 < h0 ||
        h1 > n_heads || dtype < REF_F64 || dtype > REF_BF16)
        return -1;
    for (int q = 0; q < 6; ++q)
        if (in[q] == NULL && T > 0)
            return -1;
    double r[1024], w[1024], k[1024], v[1024], a[1024], b[1024];
    for (int64_t h = h0; h < h1; ++h) {
        double *Sh = S + h * N * N;
        for (int64_t t = 0; t < T; ++t) {
            int64_t base = (t * n_heads + h) * N;
            for (int64_t c = 0; c < N; ++c) {
                r[c] = widen(in[0], dtype, base + c);
                w[c] = widen(in[1], dtype, base + c);
                k[c] = widen(in[2], dtype, base + c);
                v[c] = widen(in[3], dtype, base + c);
                a[c] = widen(in[4], dtype, base + c);
                b[c] = widen(in[5], dtype, base + c);
            }
            double *ot = o + base;
            for (int64_t i = 0; i < N; ++i) {
                double *row = Sh + i * N;
                /* delta-rule term on the state before this step's decay */
                double sa = 0.0;
                for (int64_t j = 0; j < N; ++j)
                    sa += row[j] * a[j];
                /* decay, delta-rule term, key-value outer product */
                for (int64_t j = 0; j < N; ++j)
                    row[j] = row[j] * w[j] + sa * b[j] + v[i] * k[j];
                /* readout from the updated state */
                double acc = 0.0;
                for (int64_t j = 0; j < N; ++j)
                    acc += row[j] * r[j];
                ot[i] = acc;
            }
        }
    }
    return 0;
}
