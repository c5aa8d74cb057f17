// Host-side weight preparation for the SVDQuant W4A4 linear and the INT8
// tensorwise W8A8 linear.
//
// Method sources (page title, passage):
//  "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
//  paragraph: activation outliers are moved into the weights (smoothing), the
//  hardest part of each weight is a 16-bit low-rank branch, the remainder is
//  quantized to 4 bits.
//  "SVDQuant ускоряет Krea 2 вдвое..." (ainews.so), "Решение: INT8 и W4A4":
//  INT8 tensorwise weights; low-rank branches need no calibration dataset.
//  "Diffusion Compiler" README, "Compiler" bullet: grouped INT4 weights.
//
// The truncated SVD is computed here without LAPACK: randomized block subspace
// iteration (Halko, Martinsson & Tropp, SIAM Review 2011, Alg. 4.4) with
// re-orthonormalization by classical Gram-Schmidt applied twice, followed by
// a one-sided Jacobi SVD (Hestenes 1958) of the small projected matrix.
// All of it is float64; only the stored factors are rounded to bf16.

#include "svdq.h"
#include "internal.h"

#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace svdq {

namespace {

// ---------------------------------------------------------------- threads --

int host_threads() {
    static int n = [] {
        const char *env = std::getenv("SVDQ_HOST_THREADS");
        int v = env ? std::atoi(env) : 0;
        if (v <= 0) v = (int)std::thread::hardware_concurrency();
        return std::max(1, std::min(v, 32));
    }();
    return n;
}

template <class F>
void parallel_for(int64_t begin, int64_t end, F &&fn) {
    int64_t total = end - begin;
    if (total <= 0) return;
    int nt = (int)std::min<int64_t>(host_threads(), total);
    if (nt <= 1) {
        fn(begin, end);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(nt);
    for (int t = 0; t < nt; ++t) {
        int64_t a = begin + total * t / nt;
        int64_t b = begin + total * (t + 1) / nt;
        pool.emplace_back([&fn, a, b] { fn(a, b); });
    }
    for (auto &th : pool) th.join();
}

// ------------------------------------------------------------ conversions --

inline float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline bool bf16_is_finite(uint16_t b) { return (b & 0x7F80u) != 0x7F80u; }

// Round a double to bfloat16 (8 significant bits), nearest-even, in a single
// rounding. Normal range: quantum 2^(e-7) for 2^e <= |x| < 2^(e+1); below
// bf16's smallest normal 2^-126 the quantum stays 2^-133.
uint16_t f64_to_bf16(double x) {
    if (x == 0.0 || !std::isfinite(x)) {
        float f = (float)x;
        uint32_t u;
        std::memcpy(&u, &f, 4);
        return (uint16_t)(u >> 16);
    }
    int e2;
    std::frexp(x, &e2);  // x = m * 2^e2, 0.5 <= |m| < 1
    int qexp = std::max(e2 - 8, -133);
    double scaled = std::ldexp(x, -qexp);  // exact
    double r = std::nearbyint(scaled);     // current mode: nearest-even
    double y = std::ldexp(r, qexp);
    const double bf16_max = (2.0 - std::ldexp(1.0, -7)) * std::ldexp(1.0, 127);
    if (std::fabs(y) > bf16_max) y = std::copysign(INFINITY, y);
    float f = (float)y;  // exact: y has at most 8 significant bits
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

// ------------------------------------------------------- dense kernels ---

// Y[K x b] = A[K x N] * Z[N x b]
void mul_AZ(const double *A, int K, int N, const double *Z, int b, double *Y) {
    parallel_for(0, K, [&](int64_t k0, int64_t k1) {
        std::vector<double> acc(b);
        for (int64_t k = k0; k < k1; ++k) {
            std::fill(acc.begin(), acc.end(), 0.0);
            const double *a = A + k * (int64_t)N;
            for (int n = 0; n < N; ++n) {
                double w = a[n];
                const double *z = Z + (int64_t)n * b;
                for (int c = 0; c < b; ++c) acc[c] += w * z[c];
            }
            std::memcpy(Y + k * (int64_t)b, acc.data(), sizeof(double) * b);
        }
    });
}

// Z[N x b] = A^T[N x K] * Q[K x b]
void mul_AtQ(const double *A, int K, int N, const double *Q, int b, double *Z) {
    parallel_for(0, N, [&](int64_t n0, int64_t n1) {
        int64_t w = n1 - n0;
        std::vector<double> acc(w * b, 0.0);
        for (int k = 0; k < K; ++k) {
            const double *a = A + (int64_t)k * N + n0;
            const double *q = Q + (int64_t)k * b;
            for (int64_t i = 0; i < w; ++i) {
                double v = a[i];
                double *o = acc.data() + i * b;
                for (int c = 0; c < b; ++c) o[c] += v * q[c];
            }
        }
        std::memcpy(Z + n0 * (int64_t)b, acc.data(), sizeof(double) * w * b);
    });
}

// Orthonormalize the b columns of V [rows x b] in place (classical
// Gram-Schmidt, twice). A column that collapses is replaced by zeros.
void orthonormalize(double *V, int64_t rows, int b) {
    std::vector<double> col(rows), proj(b);
    for (int j = 0; j < b; ++j) {
        for (int64_t r = 0; r < rows; ++r) col[r] = V[r * b + j];
        double norm0 = 0.0;
        for (int64_t r = 0; r < rows; ++r) norm0 += col[r] * col[r];
        norm0 = std::sqrt(norm0);
        for (int pass = 0; pass < 2; ++pass) {
            std::fill(proj.begin(), proj.end(), 0.0);
            for (int64_t r = 0; r < rows; ++r) {
                const double *row = V + r * b;
                double c = col[r];
                for (int i = 0; i < j; ++i) proj[i] += row[i] * c;
            }
            for (int64_t r = 0; r < rows; ++r) {
                const double *row = V + r * b;
                double s = 0.0;
                for (int i = 0; i < j; ++i) s += row[i] * proj[i];
                col[r] -= s;
            }
        }
        double norm = 0.0;
        for (int64_t r = 0; r < rows; ++r) norm += col[r] * col[r];
        norm = std::sqrt(norm);
        double inv = (norm > 1e-300 && norm > 1e-14 * norm0) ? 1.0 / norm : 0.0;
        for (int64_t r = 0; r < rows; ++r) V[r * b + j] = col[r] * inv;
    }
}

uint64_t splitmix64(uint64_t &s) {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Standard normal draws (Box-Muller on splitmix64 uniforms).
void gaussian_fill(double *out, int64_t n, uint64_t seed) {
    uint64_t s = seed;
    for (int64_t i = 0; i < n; i += 2) {
        double u1 = ((splitmix64(s) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
        double u2 = ((splitmix64(s) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
        double rad = std::sqrt(-2.0 * std::log(u1));
        out[i] = rad * std::cos(6.283185307179586 * u2);
        if (i + 1 < n) out[i + 1] = rad * std::sin(6.283185307179586 * u2);
    }
}

// One-sided Jacobi SVD of Z [rows x b]: rotates column pairs of Z until they
// are mutually orthogonal, accumulating the rotations in J [b x b].
// Returns false if the sweeps did not converge.
bool one_sided_jacobi(double *Z, int64_t rows, int b, double *J) {
    for (int i = 0; i < b; ++i)
        for (int j = 0; j < b; ++j) J[i * b + j] = (i == j) ? 1.0 : 0.0;
    const double tol = 1e-15;
    for (int sweep = 0; sweep < 80; ++sweep) {
        bool rotated = false;
        for (int p = 0; p < b - 1; ++p) {
            for (int q = p + 1; q < b; ++q) {
                double alpha = 0.0, beta = 0.0, gamma = 0.0;
                for (int64_t r = 0; r < rows; ++r) {
                    double zp = Z[r * b + p], zq = Z[r * b + q];
                    alpha += zp * zp;
                    beta += zq * zq;
                    gamma += zp * zq;
                }
                if (gamma == 0.0 || std::fabs(gamma) <= tol * std::sqrt(alpha * beta)) continue;
                rotated = true;
                double zeta = (beta - alpha) / (2.0 * gamma);
                double t = std::copysign(1.0, zeta) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
                double c = 1.0 / std::sqrt(1.0 + t * t);
                double s = c * t;
                for (int64_t r = 0; r < rows; ++r) {
                    double zp = Z[r * b + p], zq = Z[r * b + q];
                    Z[r * b + p] = c * zp - s * zq;
                    Z[r * b + q] = s * zp + c * zq;
                }
                for (int r = 0; r < b; ++r) {
                    double jp = J[r * b + p], jq = J[r * b + q];
                    J[r * b + p] = c * jp - s * jq;
                    J[r * b + q] = s * jp + c * jq;
                }
            }
        }
        if (!rotated) return true;
    }
    return false;
}

}  // namespace

// Top-`rank` singular triplets of A [K x N] (float64, row-major).
// U [K x rank], S [rank] (descending), V [N x rank].
svdq_status truncated_svd(const double *A, int K, int N, int rank, double *U,
                          double *S, double *V) {
    const int full = std::min(K, N);
    const int over = std::max(16, rank / 2);
    const int b = std::min(full, rank + over);
    const int iters = (b == full) ? 1 : 14;
    std::vector<double> Q((int64_t)K * b), Z((int64_t)N * b);
    gaussian_fill(Z.data(), (int64_t)N * b, 0x5EEDull + (uint64_t)K * 131 + N);
    mul_AZ(A, K, N, Z.data(), b, Q.data());
    orthonormalize(Q.data(), K, b);
    for (int it = 0; it < iters; ++it) {
        mul_AtQ(A, K, N, Q.data(), b, Z.data());
        orthonormalize(Z.data(), N, b);
        mul_AZ(A, K, N, Z.data(), b, Q.data());
        orthonormalize(Q.data(), K, b);
    }
    // B^T = A^T Q  (N x b); Jacobi on its columns: B^T J = [sigma_i v_i]
    mul_AtQ(A, K, N, Q.data(), b, Z.data());
    std::vector<double> J((int64_t)b * b);
    if (!one_sided_jacobi(Z.data(), N, b, J.data())) return SVDQ_ERR_NUMERICAL;
    std::vector<double> sig(b);
    for (int i = 0; i < b; ++i) {
        double s2 = 0.0;
        for (int64_t n = 0; n < N; ++n) s2 += Z[n * b + i] * Z[n * b + i];
        sig[i] = std::sqrt(s2);
    }
    std::vector<int> order(b);
    for (int i = 0; i < b; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return sig[x] > sig[y]; });
    for (int i = 0; i < rank; ++i) {
        int c = order[i];
        double sv = sig[c];
        if (!std::isfinite(sv)) return SVDQ_ERR_NUMERICAL;
        S[i] = sv;
        double inv = sv > 0 ? 1.0 / sv : 0.0;
        for (int64_t n = 0; n < N; ++n) V[n * rank + i] = Z[n * b + c] * inv;
        for (int64_t k = 0; k < K; ++k) {
            double u = 0.0;
            const double *q = Q.data() + k * b;
            for (int j = 0; j < b; ++j) u += q[j] * J[(int64_t)j * b + c];
            U[k * rank + i] = u;
        }
    }
    return SVDQ_OK;
}

// INT4 symmetric group quantization of one column of R (stride `ld`), one
// group of 64: A = max|r|, scale = A / 7 (fp32), q = clamp(rne(r / scale)).
static void quantize_group_int4(const float *r, int64_t ld, int n, int8_t *q,
                                float *scale) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(r[i * ld]));
    float sc = amax / 7.0f;
    *scale = sc;
    if (sc == 0.0f) {
        for (int i = 0; i < n; ++i) q[i] = 0;
        return;
    }
    for (int i = 0; i < n; ++i) {
        float quot = r[i * ld] / sc;
        float v = std::nearbyint(quot);
        v = std::min(7.0f, std::max(-7.0f, v));
        q[i] = (int8_t)v;
    }
}

// R = fp32(s_k (W - L1s L2)) as fp32 [K x N], the product summed over j in
// ascending order in float64 (each bf16 x bf16 product is exact there).
static std::vector<float> compute_residual(const uint16_t *W, int K, int N, const float *smooth,
                                           const uint16_t *l1t, const uint16_t *l2t, int rank) {
    std::vector<float> R((int64_t)K * N);
    std::vector<double> l1((int64_t)K * rank), l2((int64_t)rank * N);
    for (int j = 0; j < rank; ++j)
        for (int k = 0; k < K; ++k) l1[(int64_t)k * rank + j] = bf16_to_f32(l1t[(int64_t)j * K + k]);
    for (int n = 0; n < N; ++n)
        for (int j = 0; j < rank; ++j) l2[(int64_t)j * N + n] = bf16_to_f32(l2t[(int64_t)n * rank + j]);
    parallel_for(0, K, [&](int64_t k0, int64_t k1) {
        std::vector<double> d(N);
        for (int64_t k = k0; k < k1; ++k) {
            std::fill(d.begin(), d.end(), 0.0);
            for (int j = 0; j < rank; ++j) {
                double a = l1[k * rank + j];
                const double *b = l2.data() + (int64_t)j * N;
                for (int n = 0; n < N; ++n) d[n] = d[n] + a * b[n];
            }
            double s = smooth[k];
            const uint16_t *wrow = W + k * (int64_t)N;
            float *rrow = R.data() + k * (int64_t)N;
            for (int n = 0; n < N; ++n) {
                double diff = (double)bf16_to_f32(wrow[n]) - d[n];
                rrow[n] = (float)(s * diff);
            }
        }
    });
    return R;
}

svdq_status prepare_residual_impl(const uint16_t *W, int K, int N,
                                  const float *smooth, const uint16_t *l1t,
                                  const uint16_t *l2t, int rank, uint8_t *qw,
                                  float *sw) {
    const int G = K / SVDQ_GROUP;
    const std::vector<float> R = compute_residual(W, K, N, smooth, l1t, l2t, rank);
    parallel_for(0, N, [&](int64_t n0, int64_t n1) {
        std::vector<int8_t> codes(K);
        for (int64_t n = n0; n < n1; ++n) {
            for (int g = 0; g < G; ++g) {
                float sc;
                quantize_group_int4(R.data() + (int64_t)g * SVDQ_GROUP * N + n, N, SVDQ_GROUP,
                                    codes.data() + g * SVDQ_GROUP, &sc);
                sw[(int64_t)g * N + n] = sc;
            }
            uint8_t *row = qw + n * (int64_t)(K / 2);
            for (int j = 0; j < K / 2; ++j) {
                uint8_t lo = (uint8_t)(codes[2 * j] & 0xF);
                uint8_t hi = (uint8_t)(codes[2 * j + 1] & 0xF);
                row[j] = (uint8_t)(lo | (hi << 4));
            }
        }
    });
    return SVDQ_OK;
}

svdq_status prepare_weights_impl(const uint16_t *W, int K, int N,
                                 const float *act_absmax, float alpha, int rank,
                                 float *smooth, uint16_t *l1t, uint16_t *l2t,
                                 uint8_t *qw, float *sw, double *sigma) {
    // smoothing factors
    const double a_exp = (double)alpha;
    const double w_exp = 1.0 - (double)alpha;
    for (int k = 0; k < K; ++k) {
        double wmax = 0.0;
        const uint16_t *row = W + (int64_t)k * N;
        for (int n = 0; n < N; ++n) wmax = std::max(wmax, (double)std::fabs(bf16_to_f32(row[n])));
        double a = act_absmax[k];
        double s = 1.0;
        if (a > 0.0 && wmax > 0.0) s = std::pow(a, a_exp) / std::pow(wmax, w_exp);
        smooth[k] = (float)s;
    }
    if (rank > 0) {
        std::vector<double> A((int64_t)K * N);
        parallel_for(0, K, [&](int64_t k0, int64_t k1) {
            for (int64_t k = k0; k < k1; ++k) {
                double s = smooth[k];
                for (int n = 0; n < N; ++n)
                    A[k * (int64_t)N + n] = s * (double)bf16_to_f32(W[k * (int64_t)N + n]);
            }
        });
        std::vector<double> U((int64_t)K * rank), S(rank), V((int64_t)N * rank);
        svdq_status st = truncated_svd(A.data(), K, N, rank, U.data(), S.data(), V.data());
        if (st != SVDQ_OK) return st;
        for (int j = 0; j < rank; ++j) {
            double root = std::sqrt(S[j]);
            if (sigma) sigma[j] = S[j];
            for (int k = 0; k < K; ++k)
                l1t[(int64_t)j * K + k] = f64_to_bf16((U[(int64_t)k * rank + j] * root) / (double)smooth[k]);
            for (int n = 0; n < N; ++n)
                l2t[(int64_t)n * rank + j] = f64_to_bf16(root * V[(int64_t)n * rank + j]);
        }
    }
    return prepare_residual_impl(W, K, N, smooth, l1t, l2t, rank, qw, sw);
}

// ---- MXFP4 (OCP microscaling: FP4 E2M1 elements, E8M0 scale per 32) ----

// E2M1 code of q: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even
// mantissa (nearbyint rounds half to even, and in each binade the even
// multiple of the quantum is the even mantissa), saturating at 6; bit 3 is
// the sign, and a value that rounds to zero is +0.
static uint8_t e2m1_code(float q) {
    const float m = std::fabs(q);
    float r;
    if (m < 2.0f)
        r = std::nearbyint(2.0f * m) * 0.5f;
    else if (m < 4.0f)
        r = std::nearbyint(m);
    else
        r = std::fmin(6.0f, 2.0f * std::nearbyint(0.5f * m));
    int c = r < 2.0f ? (int)(2.0f * r) : (r < 4.0f ? (int)r + 2 : (int)(0.5f * r) + 4);
    if (c != 0 && q < 0.0f) c |= 8;
    return (uint8_t)c;
}

// One MX block of 32 values v[i * ld]: e = floor(log2 amax) - 2 clamped to
// [-127, 127] (-127 for an all-zero block); codes of v / 2^e (a power of
// two: exact, or an underflow far below E2M1's smallest step).
static int mx_block(const float *v, int64_t ld, uint8_t *codes) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(v[i * ld]));
    int e = -127;
    if (amax > 0.0f) {
        int x;
        std::frexp(amax, &x);  // amax = f 2^x, f in [0.5, 1): floor(log2 amax) = x - 1
        e = std::min(127, std::max(-127, x - 1 - 2));
    }
    const float inv = std::ldexp(1.0f, -e);
    for (int i = 0; i < 32; ++i) codes[i] = e2m1_code(v[i * ld] * inv);
    return e;
}

size_t mx_scale_ld(int rows) { return (size_t)((rows + 15) / 16 * 16); }

// Writes row r's codes of k-block kb (32 codes, nibble i at byte i / 2, low
// nibble for even i) into the MX container of `rows` rows: blocks of 128
// rows (n_b in the last), group g = kb / 2 of block b0 at b0 K/2 + g n_b 32,
// half h = kb % 2 at + h n_b 16, row r - b0 at + 16 (r - b0).
static void mx_put(uint8_t *out, int rows, int K, int r, int kb, const uint8_t *codes) {
    const int64_t b0 = (int64_t)(r / 128) * 128;
    const int64_t nb = std::min<int64_t>(128, rows - b0);
    uint8_t *dst = out + b0 * (K / 2) + (int64_t)(kb / 2) * nb * 32 + (int64_t)(kb % 2) * nb * 16 + (r - b0) * 16;
    for (int i = 0; i < 16; ++i) dst[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
}

svdq_status mx_prepare_residual_impl(const uint16_t *W, int K, int N, const float *smooth,
                                     const uint16_t *l1t, const uint16_t *l2t, int rank, uint8_t *qw,
                                     uint8_t *uw) {
    const std::vector<float> R = compute_residual(W, K, N, smooth, l1t, l2t, rank);
    const int64_t ld = (int64_t)mx_scale_ld(N);
    parallel_for(0, N, [&](int64_t n0, int64_t n1) {
        uint8_t codes[32];
        for (int64_t n = n0; n < n1; ++n)
            for (int kb = 0; kb < K / 32; ++kb) {
                const int e = mx_block(R.data() + (int64_t)kb * 32 * N + n, N, codes);
                uw[kb * ld + n] = (uint8_t)(e + 127);
                mx_put(qw, N, K, (int)n, kb, codes);
            }
    });
    return SVDQ_OK;
}

svdq_status w8a8_prepare_impl(const uint16_t *W, int K, int N, int8_t *qw, float *sw) {
    float amax = 0.0f;
    for (int64_t i = 0; i < (int64_t)K * N; ++i) amax = std::max(amax, std::fabs(bf16_to_f32(W[i])));
    float sc = amax / 127.0f;
    *sw = sc;
    parallel_for(0, N, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n) {
            for (int k = 0; k < K; ++k) {
                int8_t q = 0;
                if (sc != 0.0f) {
                    float v = std::nearbyint(bf16_to_f32(W[(int64_t)k * N + n]) / sc);
                    v = std::min(127.0f, std::max(-127.0f, v));
                    q = (int8_t)v;
                }
                qw[n * (int64_t)K + k] = q;
            }
        }
    });
    return SVDQ_OK;
}

// W4A16 container (the awq_w4a16 layer type): each column's K-groups
// quantized like the residual above, then written in units of 32 columns
// (two tiles of 16) x one pair of K-groups (128 k). Unit (b, p) holds 2 x
// 1024 bytes of codes -- tile j's slot l (16 bytes at 1024 j + 16 l) has, in
// its dword d, the codes of column 32b + 16j + l % 16 at k = 64(2p + d / 2) +
// 32(d % 2) + 8(l / 16) + i, i = 0..7, as u = q + 8 with i = 2t at bits 4t
// and i = 2t + 1 at bits 16 + 4t -- followed by 64 fp32 scales, column
// 32b + 16j + c and group 2p + e at byte 2048 + 16c + 8j + 4e. Padding
// (columns past N, the second group of an odd count): u = 8, scale 0.
size_t w4a16_container_bytes(int K, int N) {
    const size_t cpairs = (size_t)((N + 31) / 32);
    const size_t pairs = (size_t)((K / SVDQ_GROUP + 1) / 2);
    return cpairs * pairs * 2304;
}

svdq_status w4a16_prepare_impl(const uint16_t *W, int K, int N, uint8_t *packed) {
    const int G = K / SVDQ_GROUP;
    const int pairs = (G + 1) / 2;
    const int cpairs = (N + 31) / 32;
    std::vector<float> Wf((int64_t)K * N);
    for (int64_t i = 0; i < (int64_t)K * N; ++i) Wf[i] = bf16_to_f32(W[i]);
    parallel_for(0, cpairs, [&](int64_t b0, int64_t b1) {
        std::vector<int8_t> codes((size_t)32 * pairs * 128);  // [column of the pair][k, padded]
        std::vector<float> scales((size_t)32 * pairs * 2);
        for (int64_t b = b0; b < b1; ++b) {
            std::fill(codes.begin(), codes.end(), (int8_t)0);
            std::fill(scales.begin(), scales.end(), 0.0f);
            for (int c = 0; c < 32; ++c) {
                const int64_t n = 32 * b + c;
                if (n >= N) continue;
                for (int g = 0; g < G; ++g)
                    quantize_group_int4(Wf.data() + (int64_t)g * SVDQ_GROUP * N + n, N, SVDQ_GROUP,
                                        codes.data() + (size_t)c * pairs * 128 + g * SVDQ_GROUP,
                                        scales.data() + (size_t)c * pairs * 2 + g);
            }
            for (int p = 0; p < pairs; ++p) {
                uint8_t *unit = packed + ((size_t)b * pairs + p) * 2304;
                for (int j = 0; j < 2; ++j)
                    for (int l = 0; l < 64; ++l) {
                        const int c = 16 * j + l % 16;
                        for (int d = 0; d < 4; ++d) {
                            const int kb = 64 * (2 * p + d / 2) + 32 * (d % 2) + 8 * (l / 16);
                            uint32_t w = 0;
                            for (int i = 0; i < 8; ++i) {
                                const uint32_t u = (uint32_t)(codes[(size_t)c * pairs * 128 + kb + i] + 8);
                                w |= u << ((i & 1) ? 16 + 4 * (i / 2) : 4 * (i / 2));
                            }
                            std::memcpy(unit + 1024 * j + 16 * l + 4 * d, &w, 4);
                        }
                    }
                for (int c = 0; c < 16; ++c)
                    for (int j = 0; j < 2; ++j)
                        for (int e = 0; e < 2; ++e)
                            std::memcpy(unit + 2048 + 16 * c + 8 * j + 4 * e,
                                        &scales[(size_t)(16 * j + c) * pairs * 2 + 2 * p + e], 4);
            }
        }
    });
    return SVDQ_OK;
}

// Canonical INT4 nibbles -> FP6 container: each code c as FP6 E2M3 of c / 8
// (sign in bit 5, |c| in bits 0-2); the codes of half h of a group packed
// LSB-first into 24 bytes H_h; the group's 48 bytes are
// H_0[0:16] | H_1[0:16] | H_0[16:24] | H_1[16:24]. Rows go in blocks of 128
// (the last holds what is left); inside a block the groups follow one
// another, each [rows of the block][48 bytes].
svdq_status repack_codes_impl(const uint8_t *q, int rows, int K, int qfmt, uint8_t *out) {
    const int64_t in_row = K / 2;
    if (qfmt == SVDQ_QFMT_INT4) {
        std::memcpy(out, q, (size_t)rows * in_row);
        return SVDQ_OK;
    }
    const int64_t out_row = (int64_t)K / 4 * 3;
    bool bad = false;
    for (int r = 0; r < rows; ++r) {
        const uint8_t *src = q + r * in_row;
        // blocks of 128 rows, groups one after another inside a block
        const int64_t b0 = (int64_t)(r / 128) * 128;
        const int64_t nb = std::min<int64_t>(128, rows - b0);
        uint8_t *blk = out + b0 * out_row + (r - b0) * 48;
        for (int g = 0; g < K / 64; ++g) {
            uint8_t *dst = blk + (int64_t)g * nb * 48;  // group g, row r of the block
            for (int h = 0; h < 2; ++h) {
                uint64_t bits[3] = {0, 0, 0};  // the 192 bits of H_h
                for (int i = 0; i < 32; ++i) {
                    const int k = 32 * h + i;
                    const uint8_t byte = src[g * 32 + k / 2];
                    const int nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
                    const int code = nib >= 8 ? nib - 16 : nib;
                    if (code == -8) bad = true;
                    const uint64_t v = (code < 0 ? 0x20u : 0u) | (uint64_t)(code < 0 ? -code : code);
                    const int bit = 6 * i;
                    bits[bit / 64] |= v << (bit % 64);
                    if (bit % 64 > 58) bits[bit / 64 + 1] |= v >> (64 - bit % 64);
                }
                uint8_t half[24];
                for (int b = 0; b < 24; ++b) half[b] = (uint8_t)(bits[b / 8] >> (8 * (b % 8)));
                std::memcpy(dst + 16 * h, half, 16);
                std::memcpy(dst + 32 + 8 * h, half + 16, 8);
            }
        }
    }
    return bad ? SVDQ_ERR_NUMERICAL : SVDQ_OK;
}

bool all_finite_bf16(const uint16_t *p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!bf16_is_finite(p[i])) return false;
    return true;
}

}  // namespace svdq
