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
// Parity is pinned by the tests in tests/test_oracle_*.py (brute force over
// tiny rows with exact rationals, closed forms, Philox cross-checks against
// the open-source PyTorch and rocRAND engines, exact draw boundaries and a
// chi-square test).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
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

// The 64-bit uniform of one row: counter = (offset, row), key = seed.
extern "C" uint64_t oracle_uniform_u64(uint64_t seed, uint64_t row, uint64_t offset) {
    uint32_t ctr[4] = {(uint32_t)offset, (uint32_t)(offset >> 32), (uint32_t)row,
                       (uint32_t)(row >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
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
// One row, with the uniform u given explicitly.
//
// info (nullable, 10 x int64):
//   [0] k_eff  [1] P  [2] m (+inf count in the support)  [3] M_k  [4] T
//   [5] kept count (J + 1, or m for +inf rows, 0 for zero-mass rows)
//   [6] M_p  [7] t  [8] position of the token in the sorted support
//   [9] row kind: 0 normal, 1 +inf, 2 zero mass
// ---------------------------------------------------------------------------
extern "C" int oracle_sample_row(const float* row, int64_t V, int32_t top_k, float top_p,
                                 uint64_t u, int32_t* token, float* renorm, int64_t* info) {
    if (V <= 0 || row == nullptr || token == nullptr) return -1;

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
    sinfo[4] = (int64_t)T;
    sinfo[5] = kept;
    sinfo[6] = (int64_t)M_p;
    sinfo[7] = (int64_t)t;
    sinfo[8] = pos;
    if (info) std::memcpy(info, sinfo, sizeof(sinfo));
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
