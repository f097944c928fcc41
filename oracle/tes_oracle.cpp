// CPU oracle for exact top-k -> top-p truncation and inverse-CDF sampling.
//
// TEST INFRASTRUCTURE ONLY.  This file defines what the GPU sampler must
// compute; it is plain, slow and written for reading against the pages.  Only
// the test suite, the package smoke check and the CPU-baseline leg of the
// benchmark load it.  It shares no code, header, table or helper with the HIP
// sampler, and the HIP sampler never calls it.
//
// Source of the semantics: FlashInfer documentation page
// "flashinfer.cake_sampling", sections "Semantics" (strict determinism,
// NaN / Inf handling, clamps) and the description of stage 2 (sort the slab,
// keep the top-p prefix, renormalise, draw by inverse CDF).  Definitions of
// the top-k set and the nucleus: SonicSampler paper, section "Sampling
// primitives", eqs. (9) and (10).  Duplicates are resolved as a stable sort
// would (Qrita paper, section 3.3 and the exactness analysis, item (c)).
//
// Per row b, with V entries x_i (fp32) and parameters k, p:
//   1. key_i = raw bits of x_i, or 0 when x_i is NaN or has its sign bit set
//      (NaN, negative and -0.0 count as +0; +inf keeps 0x7F800000).
//   2. k_eff = V when k <= 0 or k >= V, else k.  P = round-half-even(p * 2^24)
//      clamped to [1, 2^24]; p NaN or <= 0 gives P = 1, p >= 1 gives 2^24.
//   3. S = the first k_eff indices of a stable sort by key, descending
//      (= lexsort(-prob, index)).
//   4. m = number of +inf entries in S.  If m > 0 the kept set is those m
//      entries with weight 1/m each; the draw is t = floor(u * m / 2^64).
//   5. q_j = floor(min(x_j, 1) * 2^32) (an exact integer), M_k = sum of q_j.
//   6. M_k = 0: token = smallest vocabulary index in S, renorm all zero.
//   7. T = ceil(P * M_k / 2^24); keep sorted position j while the exclusive
//      prefix mass S_excl(j) < T.  J = last kept, M_p = S_incl(J).
//   8. u = x0 | x1 << 32 of Philox4x32-10 with key (seed lo, seed hi) and
//      counter (offset lo, offset hi, row lo, row hi); t = floor(u*M_p/2^64);
//      token = S[first j with S_incl(j) > t].
//   9. renorm_out[b][S[j]] = fp32(q_j / M_p) for kept j, 0 elsewhere.
//
// Min-p (SonicSampler paper, appendix C.2, eq. (11)): with theta in (0, 1],
// the support entries whose mass q_j >= theta * q_max (q_max = the largest
// mass of the support, compared exactly) form a prefix of the sorted support;
// it is applied after top-k and top-p, as the truncation epilogue of the
// paper's stage-2 kernel lists them (TopK, TopP, MinP): the kept set is the
// shorter of the top-p prefix and the min-p prefix.  theta NaN or <= 0 turns
// it off; theta > 1 counts as 1.
//
// Logit rows (SonicSampler appendix C.1, temperature eq. (8), and the
// softmax that turns logits into probabilities): x_i = logit, NaN counts as
// -inf; M = max_i x_i.  Each entry gets the fp32 weight
//   w_i = 1                          if x_i == M,
//   w_i = E(fl(fl(x_i - M) * r))      otherwise,
// with r = fp32(fp64(1 / tau)) (tau NaN or <= 0: r = +inf, the tau -> 0
// limit; tau = +inf: r = 0) and E(s) the fp32 exponential of s <= 0 defined
// below.  Rows with M = +inf weigh their +inf entries +inf and the rest 0;
// rows with M = -inf (every entry -inf or NaN) weigh everything 0.  w is the
// row's softmax(x / tau) scaled so that its largest entry is 1, and the row is
// then sampled by steps 1-9 as a probability row (step 1 is the identity on
// w; the scale cancels in every step).
//
// Parity is pinned by the tests in tests/test_oracle_*.py (brute force over
// tiny rows with exact rationals, closed forms, Philox cross-checks against
// the open-source PyTorch and rocRAND engines, exact draw boundaries and a
// chi-square test).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <thread>
#include <vector>

typedef unsigned __int128 u128;

// ---------------------------------------------------------------------------
// Philox4x32-10.  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3" (SC'11), section 4: each round multiplies counter words 0
// and 2 by two fixed odd constants, swaps the halves of the 64-bit products
// into the other word pair and xors in the round key; the key is advanced by
// two Weyl constants (golden ratio and sqrt(3) - 1, scaled to 32 bits)
// between rounds.  Ten rounds.
// ---------------------------------------------------------------------------
static const uint32_t kPhiloxMul0 = 0xD2511F53u;
static const uint32_t kPhiloxMul1 = 0xCD9E8D57u;
static const uint32_t kPhiloxWeyl0 = 0x9E3779B9u;
static const uint32_t kPhiloxWeyl1 = 0xBB67AE85u;

static void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)kPhiloxMul0 * c[0];
    uint64_t p1 = (uint64_t)kPhiloxMul1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    uint32_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

extern "C" void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                                     uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k[0] += kPhiloxWeyl0;
            k[1] += kPhiloxWeyl1;
        }
        philox_round(c, k);
    }
    for (int i = 0; i < 4; ++i) out[i] = c[i];
}

// The Philox block of one row: counter = (offset, row), key = seed.
static void row_block(uint64_t seed, uint64_t row, uint64_t offset, uint32_t out[4]) {
    uint32_t ctr[4] = {(uint32_t)offset, (uint32_t)(offset >> 32), (uint32_t)row,
                       (uint32_t)(row >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    oracle_philox4x32_10(ctr, key, out);
}

// The 64-bit uniform of one row: words 0 and 1 of its block.
extern "C" uint64_t oracle_uniform_u64(uint64_t seed, uint64_t row, uint64_t offset) {
    uint32_t out[4];
    row_block(seed, row, offset, out);
    return (uint64_t)out[0] | ((uint64_t)out[1] << 32);
}

// ---------------------------------------------------------------------------
// Per-entry helpers.
// ---------------------------------------------------------------------------
static const uint32_t kInfBits = 0x7F800000u;

// Step 1: NaN (any payload, either sign) and anything with the sign bit set
// (-0.0, negatives, -inf) become +0.
static uint32_t sanitized_key(float x) {
    if (std::isnan(x) || std::signbit(x)) return 0u;
    uint32_t bits;
    std::memcpy(&bits, &x, 4);
    return bits;
}

static float key_value(uint32_t key) {
    float v;
    std::memcpy(&v, &key, 4);
    return v;
}

// Step 5: q = floor(min(x, 1) * 2^32), computed in double (exact: a float
// times a power of two is exact in double and floor of it is exact).
static uint64_t fixed_point_mass(uint32_t key) {
    double v = (double)key_value(key);
    if (v >= 1.0) return (uint64_t)1 << 32;
    return (uint64_t)std::floor(std::ldexp(v, 32));
}

// Step 2 (P): round-half-even of p * 2^24, clamped to [1, 2^24].
static uint64_t fixed_point_p(float p) {
    if (!(p > 0.0f)) return 1;               // NaN or p <= 0
    if (p >= 1.0f) return (uint64_t)1 << 24;  // includes +inf
    double scaled = std::ldexp((double)p, 24);  // exact
    double r = std::nearbyint(scaled);           // default rounding: half-even
    if (r < 1.0) r = 1.0;
    return (uint64_t)r;
}

static int64_t effective_k(int32_t k, int64_t V) {
    if (k <= 0 || (int64_t)k >= V) return V;
    return k;
}

// Stable sort of the indices by key, descending (ties keep ascending index),
// cut to the first k_eff: the support S in its order.
static std::vector<int64_t> support_order(const std::vector<uint32_t>& key, int64_t k_eff) {
    std::vector<int64_t> order(key.size());
    std::iota(order.begin(), order.end(), (int64_t)0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t b) { return key[a] > key[b]; });
    order.resize(k_eff);
    return order;
}

// ---------------------------------------------------------------------------
// E(s) for fp32 s <= 0: exp(s) evaluated with a fixed sequence of IEEE-754
// fp32 operations (each correctly rounded: multiply, round-to-integer ties to
// even, fused multiply-add, scaling by a power of two), so that any
// implementation that performs the same operations gets the same bits.  The
// method is Cody and Waite's argument reduction (W. J. Cody and W. Waite,
// "Software Manual for the Elementary Functions", 1980): n = rint(s / ln 2),
// f = s - n ln 2 with ln 2 split into a high and a low part, then
// exp(f) by the Taylor polynomial sum_{j<=7} f^j / j! in Horner form, and
// exp(s) = exp(f) * 2^n.  Results below 2^-125 (n < -125), NaN and s < -104
// give 0, so no result is subnormal.
// ---------------------------------------------------------------------------
static float taylor_coefficient(int j) {
    double f = 1.0;
    for (int i = 2; i <= j; ++i) f *= (double)i;
    return (float)(1.0 / f);  // the fp32 nearest 1/j! (checked exactly by the tests)
}

extern "C" float oracle_exp_weight(float s) {
    if (!(s >= -104.0f)) return 0.0f;  // NaN, -inf and far below the smallest weight
    const float log2e = 0x1.715476p+0f;     // fp32 nearest log2(e)
    const float ln2_hi = 0x1.62e43p-1f;     // fp32 nearest ln(2)
    const float ln2_lo = -0x1.05c61p-29f;   // fp32 nearest ln(2) - ln2_hi
    const float n = std::nearbyint(s * log2e);
    if (n < -125.0f) return 0.0f;
    float f = std::fma(n, -ln2_hi, s);
    f = std::fma(n, -ln2_lo, f);
    float p = taylor_coefficient(7);
    for (int j = 6; j >= 0; --j) p = std::fma(p, f, taylor_coefficient(j));
    return std::ldexp(p, (int)n);
}

// The weights w[0, V) of one logit row (see the file header).
extern "C" int oracle_logit_weights(const float* x, int64_t V, float tau, float* w) {
    if (V <= 0 || !x || !w) return -1;
    const float ninf = -std::numeric_limits<float>::infinity();
    float M = ninf;
    for (int64_t i = 0; i < V; ++i) {
        const float xi = std::isnan(x[i]) ? ninf : x[i];
        if (xi > M) M = xi;
    }
    if (M == std::numeric_limits<float>::infinity()) {
        for (int64_t i = 0; i < V; ++i) w[i] = (x[i] == M) ? M : 0.0f;
        return 0;
    }
    if (M == ninf) {
        for (int64_t i = 0; i < V; ++i) w[i] = 0.0f;
        return 0;
    }
    float r;
    if (!(tau > 0.0f)) r = std::numeric_limits<float>::infinity();
    else r = (float)(1.0 / (double)tau);  // 0 for tau = +inf
    for (int64_t i = 0; i < V; ++i) {
        const float xi = std::isnan(x[i]) ? ninf : x[i];
        if (xi == M) {
            w[i] = 1.0f;
        } else {
            const float d = xi - M;
            const float sc = d * r;
            w[i] = oracle_exp_weight(sc);
        }
    }
    return 0;
}

// ceil(theta * qmax) for theta in (0, 1], exactly: theta = m * 2^e with an
// integer m < 2^24.
static uint64_t min_p_floor_mass(float theta, uint64_t qmax) {
    int e = 0;
    const double fr = std::frexp((double)theta, &e);  // theta = fr * 2^e, fr in [0.5, 1)
    const uint64_t m = (uint64_t)std::ldexp(fr, 24);  // exact: theta has 24 bits
    e -= 24;                                           // theta = m * 2^e, e < 0 here
    const u128 prod = (u128)m * (u128)qmax;  // < 2^57
    const int sh = -e;
    if (sh >= 64) return prod != 0 ? 1 : 0;  // theta * qmax <= 2^-7: ceil is 1 (or 0)
    const u128 q = prod >> sh;
    const bool rem = (prod & (((u128)1 << sh) - 1)) != 0;
    return (uint64_t)q + (rem ? 1 : 0);
}

// ---------------------------------------------------------------------------
// One row, with the uniform u given explicitly.
//
// info (nullable, 10 x int64):
//   [0] k_eff  [1] P  [2] m (+inf count in the support)  [3] M_k  [4] T
//   [5] kept count (J + 1, or m for +inf rows, 0 for zero-mass rows)
//   [6] M_p  [7] t  [8] position of the token in the sorted support
//   [9] row kind: 0 normal, 1 +inf, 2 zero mass
// ---------------------------------------------------------------------------
// num / den (nullable): the row's final distribution as exact fractions,
// num[x] / den for every vocabulary index x (q_j / M_p on the kept entries,
// 1 / m on kept +inf entries, 1 / 1 on the token of a zero-mass row).
static int sample_row_core(const float* row, int64_t V, int32_t top_k, float top_p, float min_p,
                           uint64_t u, int32_t* token, float* renorm, int64_t* info,
                           uint64_t* num, uint64_t* den) {
    if (V <= 0 || row == nullptr || token == nullptr) return -1;
    if (num) std::fill(num, num + V, (uint64_t)0);

    std::vector<uint32_t> key(V);
    for (int64_t i = 0; i < V; ++i) key[i] = sanitized_key(row[i]);

    const int64_t k_eff = effective_k(top_k, V);
    const uint64_t P = fixed_point_p(top_p);

    // Step 3: the support S in its sorted order.
    std::vector<int64_t> order = support_order(key, k_eff);

    if (renorm) std::fill(renorm, renorm + V, 0.0f);
    int64_t inf_count = 0;
    for (int64_t j = 0; j < k_eff; ++j)
        if (key[order[j]] == kInfBits) ++inf_count;

    int64_t sinfo[10] = {k_eff, (int64_t)P, inf_count, 0, 0, 0, 0, 0, 0, 0};

    if (inf_count > 0) {
        // Step 4: +inf entries sort first; keep exactly them, uniformly.
        uint64_t t = (uint64_t)(((u128)u * (u128)inf_count) >> 64);
        *token = (int32_t)order[t];
        if (renorm) {
            float w = (float)(1.0 / (double)inf_count);
            for (int64_t j = 0; j < inf_count; ++j) renorm[order[j]] = w;
        }
        if (num) {
            for (int64_t j = 0; j < inf_count; ++j) num[order[j]] = 1;
            *den = (uint64_t)inf_count;
        }
        sinfo[5] = inf_count;
        sinfo[7] = (int64_t)t;
        sinfo[8] = (int64_t)t;
        sinfo[9] = 1;
        if (info) std::memcpy(info, sinfo, sizeof(sinfo));
        return 0;
    }

    std::vector<uint64_t> q(k_eff);
    uint64_t M_k = 0;
    for (int64_t j = 0; j < k_eff; ++j) {
        q[j] = fixed_point_mass(key[order[j]]);
        M_k += q[j];
    }
    sinfo[3] = (int64_t)M_k;

    if (M_k == 0) {
        // Step 6: smallest vocabulary index present in the support.
        *token = (int32_t)*std::min_element(order.begin(), order.end());
        if (num) {
            num[*token] = 1;
            *den = 1;
        }
        sinfo[9] = 2;
        if (info) std::memcpy(info, sinfo, sizeof(sinfo));
        return 0;
    }

    // Step 7: T = ceil(P * M_k / 2^24).
    u128 prod = (u128)P * (u128)M_k;
    uint64_t T = (uint64_t)(prod >> 24) + (((uint64_t)prod & 0xFFFFFFu) != 0 ? 1 : 0);
    int64_t kept = 0;
    uint64_t s_excl = 0;
    while (kept < k_eff && s_excl < T) {
        s_excl += q[kept];
        ++kept;
    }
    // Min-p (off for theta NaN or <= 0): the support entries with
    // q_j >= ceil(theta * q_max) are a prefix; keep the shorter prefix.
    if (min_p > 0.0f) {
        const float theta = min_p > 1.0f ? 1.0f : min_p;
        const uint64_t floor_mass = min_p_floor_mass(theta, q[0]);  // q[0] = q_max
        int64_t n_min_p = 0;
        while (n_min_p < k_eff && q[n_min_p] >= floor_mass) ++n_min_p;
        if (n_min_p < kept) {
            kept = n_min_p;
            s_excl = 0;
            for (int64_t j = 0; j < kept; ++j) s_excl += q[j];
        }
    }
    const uint64_t M_p = s_excl;  // S_incl(J)

    // Step 8: inverse CDF on the kept prefix.
    uint64_t t = (uint64_t)(((u128)u * (u128)M_p) >> 64);
    int64_t pos = 0;
    uint64_t s_incl = q[0];
    while (s_incl <= t) {
        ++pos;
        s_incl += q[pos];
    }
    *token = (int32_t)order[pos];

    // Step 9: renormalised weights of the kept entries, vocabulary order.
    if (renorm) {
        for (int64_t j = 0; j < kept; ++j)
            renorm[order[j]] = (float)((double)q[j] / (double)M_p);
    }
    if (num) {
        for (int64_t j = 0; j < kept; ++j) num[order[j]] = q[j];
        *den = M_p;
    }
    sinfo[4] = (int64_t)T;
    sinfo[5] = kept;
    sinfo[6] = (int64_t)M_p;
    sinfo[7] = (int64_t)t;
    sinfo[8] = pos;
    if (info) std::memcpy(info, sinfo, sizeof(sinfo));
    return 0;
}

extern "C" int oracle_sample_row_minp(const float* row, int64_t V, int32_t top_k, float top_p,
                                      float min_p, uint64_t u, int32_t* token, float* renorm,
                                      int64_t* info) {
    return sample_row_core(row, V, top_k, top_p, min_p, u, token, renorm, info, nullptr, nullptr);
}

extern "C" int oracle_sample_row(const float* row, int64_t V, int32_t top_k, float top_p,
                                 uint64_t u, int32_t* token, float* renorm, int64_t* info) {
    return oracle_sample_row_minp(row, V, top_k, top_p, 0.0f, u, token, renorm, info);
}

// ---------------------------------------------------------------------------
// Speculative verification (SonicSampler paper, appendix C.4, eqs. (15) and
// (16), and its draft-to-target mapping; the acceptance rule u * q(d) <= p(d)
// of section 2).  N requests, each with L draft tokens d_l drawn by a draft
// model from distributions q_l, and Lt target rows.  Draft position l (and
// the bonus position L) reads target row pi(l) of its request (pi = the
// identity when target_map is null).  With g = n * Lt + pi(l):
//   p_g     = target row g's final distribution, by steps 1-9 with its
//             top_k / top_p (num / den above);
//   q_l(x)  = Q_x / 2^32, Q_x = floor(min(y_x, 1) * 2^32) of the sanitised
//             draft probability y_x (the draft row as given, not
//             renormalised);
//   accept  d_l iff U_a * q_l(d_l) <= p_g(d_l) with U_a = u_a / 2^64, u_a =
//             x2 | x3 << 32 of the Philox block of (seed, g, offset) (words
//             0 and 1 are the row's own draw), compared exactly:
//             u_a * Q_d * den <= num[d] * 2^96;
//   on the first rejection at l, the correction token is drawn from
//             max(0, p_g - q_l) (eq. (16)) by inverse CDF in vocabulary order:
//             R_x = max(0, num[x] * 2^32 - Q_x * den), R = sum R_x,
//             t = floor(u * R / 2^64) with u = x0 | x1 << 32 of row g's
//             block, correction = the first x whose inclusive prefix of R
//             exceeds t (R = 0: row g's own token);
//   if every draft is accepted, the bonus token is the own token of target
//             row pi(L).
// out_tokens[n][0, L + 1) holds the accepted drafts, then the correction or
// the bonus, then -1; accept_len[n] = the number of accepted drafts.  A
// request whose map or draft tokens are out of range gets accept_len -1 and
// all tokens -1.
// ---------------------------------------------------------------------------
extern "C" uint64_t oracle_uniform_u64_hi(uint64_t seed, uint64_t row, uint64_t offset) {
    uint32_t out[4];
    row_block(seed, row, offset, out);
    return (uint64_t)out[2] | ((uint64_t)out[3] << 32);
}

// u * Q * den <= num * 2^96, exactly (u < 2^64, Q <= 2^32, den < 2^51, num <= 2^32).
static bool accept_draft(uint64_t u, uint64_t Q, uint64_t den, uint64_t num) {
    const u128 a = (u128)u * (u128)Q;             // < 2^96
    const uint64_t a_hi = (uint64_t)(a >> 64), a_lo = (uint64_t)a;
    const u128 lo_prod = (u128)a_lo * (u128)den;  // < 2^115
    const u128 hi = (u128)a_hi * (u128)den + (lo_prod >> 64);  // the product >> 64
    const uint64_t low = (uint64_t)lo_prod;                    // the product mod 2^64
    const u128 rhs = (u128)num << 32;                          // num * 2^96 >> 64
    return hi < rhs || (hi == rhs && low == 0);
}

extern "C" int oracle_accept_draft(uint64_t u, uint64_t Q, uint64_t den, uint64_t num) {
    return accept_draft(u, Q, den, num) ? 1 : 0;
}

extern "C" int oracle_spec_verify(const float* target, int64_t N, int64_t Lt, int64_t V,
                                  const int32_t* top_k, const float* top_p, const float* draft,
                                  int64_t L, const int32_t* draft_tokens,
                                  const int32_t* target_map, uint64_t seed, uint64_t offset,
                                  int32_t* out_tokens, int32_t* accept_len, int n_threads) {
    if (N < 0 || Lt <= 0 || V <= 0 || L < 0) return -1;
    if (N == 0) return 0;
    if (!target || !top_k || !top_p || !out_tokens || !accept_len) return -1;
    if (L > 0 && (!draft || !draft_tokens)) return -1;
    if (!target_map && Lt < L + 1) return -1;
    if (n_threads <= 0) n_threads = 1;
    if ((int64_t)n_threads > N) n_threads = (int)N;
    std::vector<int> status(n_threads, 0);
    auto work = [&](int wk) {
        std::vector<uint64_t> num(V);
        for (int64_t n = N * wk / n_threads; n < N * (wk + 1) / n_threads; ++n) {
            int32_t* out = out_tokens + n * (L + 1);
            for (int64_t l = 0; l <= L; ++l) out[l] = -1;
            accept_len[n] = -1;
            auto row_of = [&](int64_t l) {
                return target_map ? (int64_t)target_map[n * (L + 1) + l] : l;
            };
            bool valid = true;
            for (int64_t l = 0; l <= L; ++l) valid = valid && row_of(l) >= 0 && row_of(l) < Lt;
            for (int64_t l = 0; l < L; ++l)
                valid = valid && draft_tokens[n * L + l] >= 0 && draft_tokens[n * L + l] < V;
            if (!valid) continue;
            int64_t l = 0;
            for (; l <= L; ++l) {
                const int64_t g = n * Lt + row_of(l);
                const uint64_t u = oracle_uniform_u64(seed, (uint64_t)g, offset);
                int32_t tok = 0;
                uint64_t den = 0;
                int rc = sample_row_core(target + g * V, V, top_k[g], top_p[g], 0.0f, u, &tok,
                                         nullptr, nullptr, num.data(), &den);
                if (rc) {
                    status[wk] = rc;
                    break;
                }
                if (l == L) {  // every draft accepted: the bonus token
                    out[L] = tok;
                    accept_len[n] = (int32_t)L;
                    break;
                }
                const float* y = draft + (n * L + l) * V;
                const int32_t d = draft_tokens[n * L + l];
                const uint64_t Qd = fixed_point_mass(sanitized_key(y[d]));
                const uint64_t ua = oracle_uniform_u64_hi(seed, (uint64_t)g, offset);
                if (accept_draft(ua, Qd, den, num[d])) {
                    out[l] = d;
                    continue;
                }
                // Rejected: the correction from max(0, p - q), vocabulary order.
                u128 R = 0;
                std::vector<u128> r(V);
                for (int64_t x = 0; x < V; ++x) {
                    const u128 a = (u128)num[x] << 32;
                    const u128 b = (u128)fixed_point_mass(sanitized_key(y[x])) * (u128)den;
                    r[x] = a > b ? a - b : 0;
                    R += r[x];
                }
                int32_t corr = tok;
                if (R > 0) {
                    const uint64_t R_hi = (uint64_t)(R >> 64), R_lo = (uint64_t)R;
                    const u128 t = (u128)u * R_hi + (((u128)u * R_lo) >> 64);  // floor(u R / 2^64)
                    u128 acc = 0;
                    for (int64_t x = 0; x < V; ++x) {
                        acc += r[x];
                        if (acc > t) {
                            corr = (int32_t)x;
                            break;
                        }
                    }
                }
                out[l] = corr;
                accept_len[n] = (int32_t)l;
                break;
            }
        }
    };
    if (n_threads == 1) {
        work(0);
    } else {
        std::vector<std::thread> pool;
        for (int wk = 0; wk < n_threads; ++wk) pool.emplace_back(work, wk);
        for (auto& th : pool) th.join();
    }
    for (int st : status)
        if (st) return st;
    return 0;
}

// ---------------------------------------------------------------------------
// The support S of one row in its sorted order (descending probability,
// ascending index: the first k_eff entries of the stable sort of step 3),
// written to out[0, min(k_eff, cap)); returns k_eff.  This is the order in
// which the cake_sampling page ("Semantics") emits its slab.
// ---------------------------------------------------------------------------
extern "C" int64_t oracle_support(const float* row, int64_t V, int32_t top_k, int64_t cap,
                                  int32_t* out) {
    if (V <= 0 || row == nullptr || (cap > 0 && out == nullptr)) return -1;
    std::vector<uint32_t> key(V);
    for (int64_t i = 0; i < V; ++i) key[i] = sanitized_key(row[i]);
    const int64_t k_eff = effective_k(top_k, V);
    const std::vector<int64_t> order = support_order(key, k_eff);
    for (int64_t j = 0; j < k_eff && j < cap; ++j) out[j] = (int32_t)order[j];
    return k_eff;
}

// ---------------------------------------------------------------------------
// Batched entry: B rows of V entries, row-major.  Rows are split statically
// across n_threads host threads (<= 0 means one).  renorm_out and info are
// nullable; info holds 10 int64 per row.
// ---------------------------------------------------------------------------
// Batched sampling of logit rows: per row the weights of oracle_logit_weights
// (temperature[b], 1 when temperature is null), then the probability method
// with min_p[b] (off when min_p is null).  renorm_out (nullable) receives the
// renormalised kept weights, i.e. the final probabilities.
extern "C" int oracle_topk_topp_sample_logits(const float* logits, int64_t B, int64_t V,
                                              const int32_t* top_k, const float* top_p,
                                              const float* temperature, const float* min_p,
                                              uint64_t seed, uint64_t offset,
                                              int32_t* out_tokens, float* renorm_out,
                                              int64_t* info, int n_threads) {
    if (B < 0 || V <= 0) return -1;
    if (B == 0) return 0;
    if (!logits || !top_k || !top_p || !out_tokens) return -1;
    if (n_threads <= 0) n_threads = 1;
    if ((int64_t)n_threads > B) n_threads = (int)B;
    std::vector<int> status(n_threads, 0);
    auto work = [&](int wk) {
        std::vector<float> w(V);
        int64_t r0 = B * wk / n_threads, r1 = B * (wk + 1) / n_threads;
        for (int64_t b = r0; b < r1; ++b) {
            const float tau = temperature ? temperature[b] : 1.0f;
            int rc = oracle_logit_weights(logits + b * V, V, tau, w.data());
            if (!rc) {
                uint64_t u = oracle_uniform_u64(seed, (uint64_t)b, offset);
                rc = oracle_sample_row_minp(w.data(), V, top_k[b], top_p[b],
                                            min_p ? min_p[b] : 0.0f, u, out_tokens + b,
                                            renorm_out ? renorm_out + b * V : nullptr,
                                            info ? info + b * 10 : nullptr);
            }
            if (rc) status[wk] = rc;
        }
    };
    if (n_threads == 1) {
        work(0);
    } else {
        std::vector<std::thread> pool;
        for (int wk = 0; wk < n_threads; ++wk) pool.emplace_back(work, wk);
        for (auto& th : pool) th.join();
    }
    for (int st : status)
        if (st) return st;
    return 0;
}

extern "C" int oracle_topk_topp_sample(const float* probs, int64_t B, int64_t V,
                                       const int32_t* top_k, const float* top_p,
                                       uint64_t seed, uint64_t offset, int32_t* out_tokens,
                                       float* renorm_out, int64_t* info, int n_threads) {
    if (B < 0 || V <= 0) return -1;
    if (B == 0) return 0;
    if (!probs || !top_k || !top_p || !out_tokens) return -1;
    if (n_threads <= 0) n_threads = 1;
    if ((int64_t)n_threads > B) n_threads = (int)B;
    std::vector<int> status(n_threads, 0);
    auto work = [&](int w) {
        int64_t r0 = B * w / n_threads, r1 = B * (w + 1) / n_threads;
        for (int64_t b = r0; b < r1; ++b) {
            uint64_t u = oracle_uniform_u64(seed, (uint64_t)b, offset);
            int rc = oracle_sample_row(probs + b * V, V, top_k[b], top_p[b], u, out_tokens + b,
                                       renorm_out ? renorm_out + b * V : nullptr,
                                       info ? info + b * 10 : nullptr);
            if (rc) status[w] = rc;
        }
    };
    if (n_threads == 1) {
        work(0);
    } else {
        std::vector<std::thread> pool;
        for (int w = 0; w < n_threads; ++w) pool.emplace_back(work, w);
        for (auto& th : pool) th.join();
    }
    for (int s : status)
        if (s) return s;
    return 0;
}
