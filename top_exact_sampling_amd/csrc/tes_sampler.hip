// Exact top-k -> top-p sampling over fp32 probability rows, for MI355X (gfx950).
//
// What is computed (FlashInfer "cake_sampling" documentation page, section
// "Semantics", and its stage-2 description): per row, the support is the first
// k entries of lexsort(-prob, index); NaN / negative / -0.0 count as +0; rows
// whose support holds +inf entries keep exactly those at weight 1/m; other
// rows keep the shortest sorted prefix whose 2^-32 fixed-point mass reaches
// round(p * 2^24) / 2^24 of the top-k mass, renormalise it and draw one token
// by inverse CDF from Philox4x32-10(seed, row, offset).  All decisions are
// integer arithmetic on exact masses, so every internal path gives bitwise
// identical results.
//
// Design (one workgroup of 1024 threads per row):
//   * Every entry becomes a 64-bit composite (key << 32) | ~index, key = the
//     sanitised fp32 bits.  Composites are unique and order entries exactly as
//     the stable descending sort does.
//   * Candidate buffer.  The row is streamed once with 16-byte loads, eight
//     loads in flight per thread.  An entry whose composite is >= a running
//     threshold theta is appended to an LDS buffer (wave ballot + one LDS
//     atomic per wave).  After each group of eight rounds one barrier checks
//     the fill; a radix select over the buffer's 11-bit composite digits
//     (LDS histograms) then compacts it to at least the best L entries and
//     raises theta.  Nothing below theta can re-enter the best L, so one read
//     leaves every entry >= theta in LDS.  This takes the place of the
//     2048-bucket radix select and candidate list of the cake_sampling page,
//     as a running filter instead of a sampled bound.
//   * k <= 1024: weighted radix selects over the buffer (exact u64 mass
//     histograms per digit) give the k-th composite, the top-p boundary and
//     the drawn entry; the support is never sorted.
//   * k >= V (top-p only): the same stream keeps the best >= 1024 entries and
//     also builds an exact mass histogram over 1/128-octave key bins (every
//     key with a nonzero mass falls in one of 4097 bins).  If the buffered
//     prefix already holds the top-p mass the row is finished in LDS (a
//     truncation hit, the exact analogue of the Gaussian sigma-truncation of
//     the Qrita paper, section 3.1).  Otherwise the histogram names the bin of
//     the boundary and the bins the draw can fall in, one more pass gathers
//     just those bins, and the selects finish in LDS.
//   * 1024 < k < V rows, and rows that defeat the above (more +inf entries
//     than buffered, over-full bins), use a multi-pass whole-row radix select.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>
#include <new>

#include "tes_sampler.h"

typedef uint64_t u64;
typedef uint32_t u32;

namespace {

constexpr int kBlock = 1024;            // threads per workgroup (16 waves)
constexpr int kWaves = kBlock / 64;
constexpr int kCap = 8192;              // candidate buffer entries (64 KiB of LDS)
constexpr int kBins = 2048;             // 11-bit radix digits
constexpr u32 kSlabMaxK = 1024;         // largest k served by the candidate buffer
constexpr u32 kFullKeep = 1024;         // best entries always kept for top-p-only rows
constexpr u32 kInfKey = 0x7F800000u;
constexpr u32 kOneKey = 0x3F800000u;    // 1.0f: masses saturate at 2^32 from here
constexpr u32 kMinMassKey = 95u << 23;  // 2^-32: the smallest value with a nonzero mass
constexpr int kFineShift = 16;          // fine bins: exponent + 7 mantissa bits
constexpr u32 kFineBase = kMinMassKey >> kFineShift;
constexpr int kFineBins = (int)((kOneKey >> kFineShift) - kFineBase) + 1;  // 4097
constexpr int kGroup = 8;               // rounds per group = loads in flight per thread
constexpr u32 kSoftFill = kCap / 2;     // compact when a group leaves more than this
constexpr u64 kNoUpper = ~0ull;

enum RowKind : u32 { kNormal = 0, kInfRow = 1, kZeroRow = 2 };
enum RowPath : u32 { kPathBuffer = 0, kPathHit = 1, kPathGather = 2, kPathRowSelect = 3 };

struct Smem {
    u64 buf[kCap];
    u64 hfine[kFineBins];
    u64 hmass[kBins];
    u32 hcnt[kBins];
    u64 wpart[kWaves];
    u64 bc[4];
    u64 theta;
    u32 gctr[3];
    u32 rctr;
    u32 ccount;
};

struct Sel {
    u64 c;      // selected composite
    u64 above;  // weight of the considered entries strictly above it
};

struct Outcome {
    u32 token;
    u32 kind;
    u64 c_keep;  // kept entries are those with composite >= c_keep
    u64 M_p;     // kept mass (normal rows)
    u32 m;       // number of kept +inf entries (inf rows)
    u32 path;
    u32 passes;
    u32 compactions;
    u32 gathered;
};

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------

// +0 for NaN and for anything with the sign bit set; otherwise the raw bits.
__device__ __forceinline__ u32 sanitize(u32 bits) { return bits <= kInfKey ? bits : 0u; }

__device__ __forceinline__ u64 composite(u32 key, u32 idx) {
    return ((u64)key << 32) | (u64)(~idx);
}

__device__ __forceinline__ u32 comp_index(u64 c) { return ~(u32)c; }

// floor(min(x, 1) * 2^32) for the non-negative float whose bits are `key`.
// x * 2^32 is exact in fp32 and the conversion truncates, i.e. floors.
__device__ __forceinline__ u64 key_mass(u32 key) {
    if (key >= kOneKey) return 1ull << 32;
    return (u64)(u32)(__uint_as_float(key) * 4294967296.0f);
}

// Fine mass bin of a key >= kMinMassKey; bins ascend with the key.
__device__ __forceinline__ u32 fine_bin(u32 key) {
    return key >= kOneKey ? (u32)(kFineBins - 1) : (key >> kFineShift) - kFineBase;
}

// Composite range [lo, hi) covered by fine bin b.
__device__ __forceinline__ u64 fine_lo(int b) {
    return (u64)((u32)(b + kFineBase) << kFineShift) << 32;
}
__device__ __forceinline__ u64 fine_hi(int b) {
    return b == kFineBins - 1 ? kNoUpper : fine_lo(b + 1);
}

// round-half-even(p * 2^24) clamped to [1, 2^24]; NaN and p <= 0 give 1.
__device__ __forceinline__ u64 fixed_p(float p) {
    if (!(p > 0.0f)) return 1;
    if (p >= 1.0f) return 1ull << 24;
    float r = rintf(p * 16777216.0f);
    u64 P = (u64)r;
    return P < 1 ? 1 : P;
}

// ceil(P * M / 2^24) with a 128-bit product.
__device__ __forceinline__ u64 topp_threshold(u64 P, u64 M) {
    u64 lo = P * M, hi = __umul64hi(P, M);
    u64 T = (hi << 40) | (lo >> 24);
    return T + ((lo & 0xFFFFFFull) != 0);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): key (seed lo, seed hi),
// counter (offset lo, offset hi, row lo, row hi); returns word0 | word1 << 32.
__device__ u64 philox_uniform(u64 seed, u64 row, u64 offset) {
    u32 x0 = (u32)offset, x1 = (u32)(offset >> 32), x2 = (u32)row, x3 = (u32)(row >> 32);
    u32 k0 = (u32)seed, k1 = (u32)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const u32 a = 0xD2511F53u, b = 0xCD9E8D57u;
        u32 lo_a = a * x0, hi_a = __umulhi(a, x0);
        u32 lo_b = b * x2, hi_b = __umulhi(b, x2);
        u32 n0 = hi_b ^ x1 ^ k0;
        u32 n2 = hi_a ^ x3 ^ k1;
        x0 = n0;
        x1 = lo_b;
        x2 = n2;
        x3 = lo_a;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return (u64)x0 | ((u64)x1 << 32);
}

// ---------------------------------------------------------------------------
// Wave / block primitives (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32 lane_id() { return threadIdx.x & 63u; }
__device__ __forceinline__ u32 wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ u32 mbcnt64(u64 m) {
    return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, 0u));
}

__device__ __forceinline__ u64 wave_sum(u64 v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ u64 wave_min(u64 v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        u64 w = __shfl_xor(v, o, 64);
        v = w < v ? w : v;
    }
    return v;
}

__device__ u64 block_sum(Smem& s, u64 v) {
    v = wave_sum(v);
    if (lane_id() == 0) s.wpart[wave_id()] = v;
    __syncthreads();
    u64 t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += s.wpart[w];
    __syncthreads();
    return t;
}

__device__ u64 block_min(Smem& s, u64 v) {
    v = wave_min(v);
    if (lane_id() == 0) s.wpart[wave_id()] = v;
    __syncthreads();
    u64 t = ~0ull;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t = s.wpart[w] < t ? s.wpart[w] : t;
    __syncthreads();
    return t;
}

__device__ u64 block_excl_scan(Smem& s, u64 v) {
    u64 x = v;
    const u32 lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        u64 y = __shfl_up(x, o, 64);
        if (lane >= (u32)o) x += y;
    }
    if (lane == 63) s.wpart[wave_id()] = x;
    __syncthreads();
    u64 pre = 0;
    const u32 w0 = wave_id();
    for (u32 w = 0; w < w0; ++w) pre += s.wpart[w];
    __syncthreads();
    return pre + x - v;
}

// Append `c` at s.buf[base + slot] for every lane with pred set; slots come
// from one LDS atomic per wave on *ctr.  Slots at or beyond `cap` are counted
// but not written.  Must be reached by whole waves.
__device__ __forceinline__ void wave_append(Smem& s, bool pred, u64 c, u32* ctr, u32 base,
                                            u32 cap = kCap) {
    u64 m = __ballot(pred);
    if (m == 0) return;
    const int leader = __ffsll((unsigned long long)m) - 1;
    u32 pos0 = 0;
    if ((int)lane_id() == leader) pos0 = atomicAdd(ctr, (u32)__popcll(m));
    pos0 = __shfl(pos0, leader, 64);
    const u32 pos = base + pos0 + mbcnt64(m);
    if (pred && pos < cap) s.buf[pos] = c;
}

// ---------------------------------------------------------------------------
// Histogram search
// ---------------------------------------------------------------------------
struct Digit {
    u32 d;
    u32 cnt;
    u64 above;
};

// Bins [0, nb) taken in descending order: the bin where the cumulative weight
// first reaches W (1 <= W <= total weight); `above` = weight of higher bins.
template <typename H>
__device__ Digit find_desc(Smem& s, int nb, u64 W, H weight) {
    const int per = (nb + kBlock - 1) / kBlock;
    const int top = nb - 1 - (int)threadIdx.x * per;
    u64 local = 0;
    for (int j = 0; j < per; ++j)
        if (top - j >= 0) local += weight(top - j);
    if (threadIdx.x == 0) {
        s.bc[0] = 0;
        s.bc[1] = 0;
    }
    u64 acc = block_excl_scan(s, local);
    for (int j = 0; j < per; ++j) {
        const int b = top - j;
        if (b >= 0) {
            const u64 w = weight(b);
            if (acc < W && W <= acc + w) {
                s.bc[0] = (u64)b;
                s.bc[1] = acc;
            }
            acc += w;
        }
    }
    __syncthreads();
    Digit g;
    g.d = (u32)s.bc[0];
    g.above = s.bc[1];
    g.cnt = 0;
    __syncthreads();
    return g;
}

__device__ __forceinline__ int level_shift(int l) { return l < 5 ? 52 - 11 * l : 0; }
__device__ __forceinline__ int level_width(int l) { return l < 5 ? 11 : 8; }
__device__ __forceinline__ u64 level_high_mask(int l) {
    int top = level_shift(l) + level_width(l);
    return top >= 64 ? 0ull : (~0ull << top);
}

// Weighted radix select over the entries c of s.buf[base, base + n) with
// lo <= c < hi: the composite at which the descending cumulative weight (one
// per entry, or its mass) first reaches W (1 <= W <= total).
__device__ Sel select_buffer(Smem& s, u32 base, u32 n, u64 W, bool mass, u64 lo, u64 hi) {
    u64 prefix = 0, above = 0;
    for (int l = 0; l < 6; ++l) {
        const int sh = level_shift(l), wd = level_width(l);
        const u64 hm = level_high_mask(l);
        const u32 dmask = (1u << wd) - 1;
        for (int b = threadIdx.x; b < (1 << wd); b += kBlock) {
            s.hcnt[b] = 0;
            s.hmass[b] = 0;
        }
        __syncthreads();
        for (u32 i = threadIdx.x; i < n; i += kBlock) {
            const u64 c = s.buf[base + i];
            if (c >= lo && c < hi && (c & hm) == prefix) {
                const u32 d = (u32)(c >> sh) & dmask;
                atomicAdd(&s.hcnt[d], 1u);
                if (mass) atomicAdd((unsigned long long*)&s.hmass[d],
                                    (unsigned long long)key_mass((u32)(c >> 32)));
            }
        }
        __syncthreads();
        Digit g = mass ? find_desc(s, 1 << wd, W - above, [&](int b) { return s.hmass[b]; })
                       : find_desc(s, 1 << wd, W - above, [&](int b) { return (u64)s.hcnt[b]; });
        g.cnt = s.hcnt[g.d];
        above += g.above;
        prefix |= (u64)g.d << sh;
        if (g.cnt == 1 || l == 5) {
            const u64 m2 = ~0ull << sh;
            for (u32 i = threadIdx.x; i < n; i += kBlock) {
                const u64 c = s.buf[base + i];
                if (c >= lo && c < hi && (c & m2) == prefix) s.bc[2] = c;
            }
            __syncthreads();
            Sel r{s.bc[2], above};
            __syncthreads();
            return r;
        }
    }
    return Sel{0, 0};  // not reached
}

// Keep at least the best L of s.buf[0..n) (n > L), choosing a radix
// threshold that leaves at most keep_max >= L entries; raises s.theta.
__device__ __noinline__ u32 compact_buffer(Smem& s, u32 n, u32 L, u32 keep_max) {
    u64 prefix = 0;
    u32 above = 0;
    for (int l = 0; l < 6; ++l) {
        const int sh = level_shift(l), wd = level_width(l);
        const u64 hm = level_high_mask(l);
        const u32 dmask = (1u << wd) - 1;
        for (int b = threadIdx.x; b < (1 << wd); b += kBlock) s.hcnt[b] = 0;
        __syncthreads();
        for (u32 i = threadIdx.x; i < n; i += kBlock) {
            const u64 c = s.buf[i];
            if ((c & hm) == prefix) atomicAdd(&s.hcnt[(u32)(c >> sh) & dmask], 1u);
        }
        __syncthreads();
        Digit g = find_desc(s, 1 << wd, (u64)(L - above), [&](int b) { return (u64)s.hcnt[b]; });
        g.cnt = s.hcnt[g.d];
        above += (u32)g.above;
        prefix |= (u64)g.d << sh;
        if (above + g.cnt <= keep_max) break;
    }
    constexpr int kPer = kCap / kBlock;
    u64 mine[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const u32 i = threadIdx.x + j * kBlock;
        mine[j] = i < n ? s.buf[i] : 0ull;
    }
    if (threadIdx.x == 0) s.ccount = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const u32 i = threadIdx.x + j * kBlock;
        wave_append(s, i < n && mine[j] >= prefix, mine[j], &s.ccount, 0);
    }
    __syncthreads();
    const u32 kept = s.ccount;
    if (threadIdx.x == 0 && prefix > s.theta) s.theta = prefix;
    __syncthreads();
    return kept;
}

// ---------------------------------------------------------------------------
// Streaming pass
// ---------------------------------------------------------------------------
template <int VEC>
struct VecT;
template <>
struct VecT<4> {
    typedef float4 T;
    __device__ static float get(const float4& v, int e) {
        return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    }
};
template <>
struct VecT<1> {
    typedef float T;
    __device__ static float get(const float& v, int) { return v; }
};

// Re-run the candidate filter over rounds [ra, rb) one round at a time,
// compacting before any round that could overflow the buffer.  Used for the
// first group of a row (theta still 0) and for a group whose appends did not
// fit; the mass histogram is not touched here.
struct Fill {
    u32 fill;
    u32 compactions;
};

template <int VEC>
__device__ __noinline__ Fill replay_rounds(Smem& s, const typename VecT<VEC>::T* __restrict__ rv,
                                           u32 nvec, u32 ra, u32 rb, u32 L, u32 keep_max,
                                           u32 fill) {
    u32 compactions = 0;
    typedef typename VecT<VEC>::T VT;
    constexpr u32 kRound = kBlock * VEC;
    for (u32 rr = ra; rr < rb; ++rr) {
        if (fill > kCap - kRound) {
            fill = compact_buffer(s, fill, L, keep_max);
            ++compactions;
        }
        const u64 theta = s.theta;
        if (threadIdx.x == 0) s.rctr = 0;
        __syncthreads();
        const u32 iv = rr * kBlock + threadIdx.x;
        const bool valid = iv < nvec;
        const VT x = valid ? rv[iv] : VT{};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const u64 c = composite(sanitize(__float_as_uint(VecT<VEC>::get(x, e))), iv * VEC + e);
            wave_append(s, valid && c >= theta, c, &s.rctr, fill);
        }
        __syncthreads();
        fill += s.rctr;
        __syncthreads();
    }
    return Fill{fill, compactions};
}

// One read of the row.  Leaves in s.buf[0, fill) every entry whose composite
// is >= s.theta (plus possibly some below it), at least the row's best
// min(L, V) entries; with FULL also the exact fine mass histogram s.hfine.
template <int VEC, bool FULL>
__device__ Fill stream_row(Smem& s, const float* __restrict__ row, u32 V, u32 L, u32 keep_max) {
    u32 compactions = 0;
    typedef typename VecT<VEC>::T VT;
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row);
    const u32 nvec = V / VEC;
    const u32 nr = (nvec + kBlock - 1) / kBlock;
    const u32 last = nvec - 1;
    const u32 tid = threadIdx.x;
    u32 fill = 0;
    u64 theta = 0;

    // pf[d] holds round g * kGroup + d.  The loads of group g + 1 are issued
    // slot by slot while group g is processed; iteration g = -1 only issues
    // the first group, so every load sits at one program point and the
    // registers of a slot never move.
    constexpr u32 kRound = kBlock * VEC;
    VT pf[kGroup];
    const int ngroups = (int)((nr + kGroup - 1) / kGroup);
    for (int g = -1; g < ngroups; ++g) {
        const u32 r0 = (u32)g * kGroup;
        u32* ctr = &s.gctr[(u32)(g + 3) % 3];
        // Group 0 starts from theta = 0: it appends round by round, compacting
        // whenever a round could overflow.  Later groups append freely and
        // check the fill once, at the group barrier.
        const bool careful = g == 0;
#pragma unroll
        for (int d = 0; d < kGroup; ++d) {
            if (g >= 0) {
                const u32 iv = (r0 + d) * kBlock + tid;
                const bool valid = iv < nvec;
                u64 c[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const u32 key = sanitize(__float_as_uint(VecT<VEC>::get(pf[d], e)));
                    if (FULL && valid && key >= kMinMassKey)
                        atomicAdd((unsigned long long*)&s.hfine[fine_bin(key)],
                                  (unsigned long long)key_mass(key));
                    c[e] = composite(key, iv * VEC + e);
                }
                if (careful) {
                    if (fill > kCap - kRound) {
                        fill = compact_buffer(s, fill, L, keep_max);
                        ++compactions;
                    }
                    theta = s.theta;
                    if (tid == 0) s.rctr = 0;
                    __syncthreads();
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        wave_append(s, valid && c[e] >= theta, c[e], &s.rctr, fill);
                    __syncthreads();
                    fill += s.rctr;
                    __syncthreads();
                } else {
                    bool pass[VEC];
                    bool any = false;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        pass[e] = valid && c[e] >= theta;
                        any |= pass[e];
                    }
                    if (__ballot(any)) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) wave_append(s, pass[e], c[e], ctr, fill);
                    }
                }
            }
            pf[d] = rv[min((u32)(g + 1) * kGroup * kBlock + d * kBlock + tid, last)];
        }
        if (g < 0) continue;
        if (!careful) {
            __syncthreads();
            const u32 napp = *ctr;
            if (fill + napp > (u32)kCap) {
                // Some appends did not fit: redo this group round by round.
                const Fill f = replay_rounds<VEC>(s, rv, nvec, r0, min(r0 + kGroup, nr), L,
                                                  keep_max, fill);
                fill = f.fill;
                compactions += f.compactions;
            } else {
                fill += napp;
            }
        }
        // The counter of group g + 2 was last used by group g - 1, whose count
        // every thread read before this group's barrier.
        if (tid == 0) s.gctr[(u32)(g + 2) % 3] = 0;
        if (fill > kSoftFill) {
            fill = compact_buffer(s, fill, L, keep_max);
            ++compactions;
        }
        theta = s.theta;
    }
    return Fill{fill, compactions};
}

// ---------------------------------------------------------------------------
// Whole-row passes
// ---------------------------------------------------------------------------
// Calls f(key, idx, valid) for every element, VEC per thread per round; every
// thread makes the same number of calls, so f may use wave collectives.  Loads
// run kGroup rounds ahead.
template <int VEC, typename F>
__device__ void for_each_entry(const float* __restrict__ row, u32 V, F f) {
    typedef typename VecT<VEC>::T VT;
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row);
    const u32 nvec = V / VEC;
    const u32 nr = (nvec + kBlock - 1) / kBlock;
    const u32 last = nvec - 1;
    VT pf[kGroup];
#pragma unroll
    for (int d = 0; d < kGroup; ++d) pf[d] = rv[min(d * kBlock + threadIdx.x, last)];
    for (u32 r0 = 0; r0 < nr; r0 += kGroup) {
#pragma unroll
        for (int d = 0; d < kGroup; ++d) {
            const u32 iv = (r0 + d) * kBlock + threadIdx.x;
            const bool valid = iv < nvec;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                f(sanitize(__float_as_uint(VecT<VEC>::get(pf[d], e))), iv * VEC + e, valid);
            pf[d] = rv[min((r0 + d + kGroup) * kBlock + threadIdx.x, last)];
        }
    }
}

// Weighted radix select over the entries of the row with composite >= lo:
// histogram one 11-bit digit per pass; once the selected bucket holds at most
// gather_cap entries, gather it into LDS and finish there.
template <int VEC>
__device__ Sel select_row(Smem& s, const float* row, u32 V, u64 W, bool mass, u64 lo,
                          u32 gather_cap, u32& passes) {
    u64 prefix = 0, above = 0;
    for (int l = 0; l < 6; ++l) {
        const int sh = level_shift(l), wd = level_width(l);
        const u64 hm = level_high_mask(l);
        const u32 dmask = (1u << wd) - 1;
        for (int b = threadIdx.x; b < kBins; b += kBlock) {
            s.hcnt[b] = 0;
            s.hmass[b] = 0;
        }
        __syncthreads();
        for_each_entry<VEC>(row, V, [&](u32 key, u32 idx, bool valid) {
            const u64 c = composite(key, idx);
            if (valid && c >= lo && (c & hm) == prefix) {
                const u32 d = (u32)(c >> sh) & dmask;
                atomicAdd(&s.hcnt[d], 1u);
                if (mass) atomicAdd((unsigned long long*)&s.hmass[d],
                                    (unsigned long long)key_mass(key));
            }
        });
        ++passes;
        __syncthreads();
        Digit g = mass ? find_desc(s, 1 << wd, W - above, [&](int b) { return s.hmass[b]; })
                       : find_desc(s, 1 << wd, W - above, [&](int b) { return (u64)s.hcnt[b]; });
        g.cnt = s.hcnt[g.d];
        above += g.above;
        prefix |= (u64)g.d << sh;
        const u64 m2 = ~0ull << sh;
        if (g.cnt <= gather_cap || l == 5) {
            if (threadIdx.x == 0) s.ccount = 0;
            __syncthreads();
            for_each_entry<VEC>(row, V, [&](u32 key, u32 idx, bool valid) {
                const u64 c = composite(key, idx);
                wave_append(s, valid && c >= lo && (c & m2) == prefix, c, &s.ccount, 0);
            });
            ++passes;
            __syncthreads();
            const u32 n = s.ccount;
            __syncthreads();
            Sel r = select_buffer(s, 0, n, W - above, mass, 0, kNoUpper);
            return Sel{r.c, above + r.above};
        }
    }
    return Sel{0, 0};  // not reached
}

// Exact resolution of a row from whole-row passes only.
template <int VEC>
__device__ void resolve_row(Smem& s, const float* row, u32 V, u32 k_eff, u64 P, u64 u,
                            u32 gather_cap, Outcome& o) {
    u64 lo = 0;
    if (k_eff < V) lo = select_row<VEC>(s, row, V, k_eff, false, 0, gather_cap, o.passes).c;
    u64 mk = 0, ninf = 0, minidx = ~0ull;
    for_each_entry<VEC>(row, V, [&](u32 key, u32 idx, bool valid) {
        if (valid && composite(key, idx) >= lo) {
            mk += key_mass(key);
            ninf += key == kInfKey;
            minidx = idx < minidx ? idx : minidx;
        }
    });
    ++o.passes;
    const u64 M_k = block_sum(s, mk);
    const u64 m = block_sum(s, ninf);
    minidx = block_min(s, minidx);
    if (m > 0) {
        const u64 t = __umul64hi(u, m);
        o.kind = kInfRow;
        o.m = (u32)m;
        o.token = comp_index(select_row<VEC>(s, row, V, t + 1, false, 0, gather_cap, o.passes).c);
        o.c_keep = select_row<VEC>(s, row, V, m, false, 0, gather_cap, o.passes).c;
        return;
    }
    if (M_k == 0) {
        o.kind = kZeroRow;
        o.token = (u32)minidx;
        return;
    }
    const u64 T = topp_threshold(P, M_k);
    const Sel bt = select_row<VEC>(s, row, V, T, true, lo, gather_cap, o.passes);
    const u64 M_p = bt.above + key_mass((u32)(bt.c >> 32));
    const u64 t = __umul64hi(u, M_p);
    const Sel dr = select_row<VEC>(s, row, V, t + 1, true, lo, gather_cap, o.passes);
    o.kind = kNormal;
    o.c_keep = bt.c;
    o.M_p = M_p;
    o.token = comp_index(dr.c);
}

// Counts, masses and the smallest index over buffered entries c >= lo.
struct BufStats {
    u64 n, ninf, mass, minidx;
};

__device__ BufStats buffer_stats(Smem& s, u32 fill, u64 lo) {
    u64 n = 0, ninf = 0, q = 0, mi = ~0ull;
    for (u32 i = threadIdx.x; i < fill; i += kBlock) {
        const u64 c = s.buf[i];
        if (c >= lo) {
            const u32 key = (u32)(c >> 32);
            ++n;
            ninf += key == kInfKey;
            q += key_mass(key);
            const u64 id = comp_index(c);
            mi = id < mi ? id : mi;
        }
    }
    BufStats r;
    r.n = block_sum(s, n);
    r.ninf = block_sum(s, ninf);
    r.mass = block_sum(s, q);
    r.minidx = block_min(s, mi);
    return r;
}

// Resolve from the buffered prefix {c >= lo} (a prefix of the row's sorted
// order).  `support_complete`: the prefix is the whole support (k <= 1024
// rows) and M_k is its mass; otherwise M_k is given (top-p-only rows) and
// the function returns false when the prefix cannot decide.
__device__ bool resolve_prefix(Smem& s, u32 fill, u64 lo, const BufStats& st,
                               bool support_complete, u64 M_k, u64 P, u64 u, Outcome& o) {
    if (st.ninf > 0) {
        if (!support_complete && st.ninf == st.n) return false;  // more +inf may lie below
        const u64 m = st.ninf;
        const u64 t = __umul64hi(u, m);
        o.kind = kInfRow;
        o.m = (u32)m;
        o.token = comp_index(select_buffer(s, 0, fill, t + 1, false, lo, kNoUpper).c);
        o.c_keep = select_buffer(s, 0, fill, m, false, lo, kNoUpper).c;
        return true;
    }
    if (M_k == 0) {
        o.kind = kZeroRow;
        o.token = support_complete ? (u32)st.minidx : 0u;  // a top-p-only support starts at 0
        return true;
    }
    const u64 T = topp_threshold(P, M_k);
    if (st.mass < T) return false;
    const Sel bt = select_buffer(s, 0, fill, T, true, lo, kNoUpper);
    const u64 M_p = bt.above + key_mass((u32)(bt.c >> 32));
    const u64 t = __umul64hi(u, M_p);
    const Sel dr = select_buffer(s, 0, fill, t + 1, true, lo, kNoUpper);
    o.kind = kNormal;
    o.c_keep = bt.c;
    o.M_p = M_p;
    o.token = comp_index(dr.c);
    return true;
}

// Top-p-only row whose nucleus is larger than the buffered prefix: the fine
// histogram names the boundary bin and the bins the draw can fall in; one
// pass gathers those bins into s.buf[fill, kCap) and the selects finish
// there.  Returns false if the gathered entries do not fit.
template <int VEC>
__device__ bool resolve_gather(Smem& s, const float* row, u32 V, u32 fill, u64 M, u64 P, u64 u,
                               Outcome& o) {
    const u64 T = topp_threshold(P, M);
    auto hw = [&](int b) { return s.hfine[b]; };
    const Digit bT = find_desc(s, kFineBins, T, hw);
    const u64 hT = s.hfine[bT.d];
    // M_p lies in [T, above(bT) + mass(bT)], so t lies in [t_lo, t_hi].
    const u64 t_lo = __umul64hi(u, T);
    const u64 t_hi = __umul64hi(u, bT.above + hT);
    const Digit bDhi = find_desc(s, kFineBins, t_lo + 1, hw);  // bin holding position t_lo
    const Digit bDlo = find_desc(s, kFineBins, t_hi + 1, hw);  // bin holding position t_hi
    const u32 bt = bT.d, dlo = bDlo.d, dhi = bDhi.d;
    if (threadIdx.x == 0) s.ccount = 0;
    __syncthreads();
    const u32 cap = kCap - fill;
    for_each_entry<VEC>(row, V, [&](u32 key, u32 idx, bool valid) {
        bool take = false;
        if (valid && key >= kMinMassKey) {
            const u32 b = fine_bin(key);
            take = b == bt || (b >= dlo && b <= dhi);
        }
        wave_append(s, take, composite(key, idx), &s.ccount, fill, kCap);
    });
    ++o.passes;
    __syncthreads();
    const u32 ng = s.ccount;
    __syncthreads();
    o.gathered = ng;
    if (ng > cap) return false;
    const Sel sb = select_buffer(s, fill, ng, T - bT.above, true, fine_lo(bt), fine_hi(bt));
    const u64 M_p = bT.above + sb.above + key_mass((u32)(sb.c >> 32));
    const u64 t = __umul64hi(u, M_p);
    const Digit bD = find_desc(s, kFineBins, t + 1, hw);
    const Sel sd = select_buffer(s, fill, ng, t + 1 - bD.above, true, fine_lo(bD.d),
                                 fine_hi(bD.d));
    o.kind = kNormal;
    o.c_keep = sb.c;
    o.M_p = M_p;
    o.token = comp_index(sd.c);
    return true;
}

template <int VEC>
__device__ void write_renorm(const float* __restrict__ row, float* __restrict__ out, u32 V,
                             const Outcome& o) {
    typedef typename VecT<VEC>::T VT;
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row);
    VT* __restrict__ ov = reinterpret_cast<VT*>(out);
    const u32 nvec = V / VEC;
    const double inv = o.kind == kNormal ? 1.0 / (double)o.M_p : 0.0;
    const float w_inf = o.kind == kInfRow ? (float)(1.0 / (double)o.m) : 0.0f;
    for (u32 iv = threadIdx.x; iv < nvec; iv += kBlock) {
        const VT x = rv[iv];
        float r[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const u32 key = sanitize(__float_as_uint(VecT<VEC>::get(x, e)));
            const bool kept = o.kind != kZeroRow && composite(key, iv * VEC + e) >= o.c_keep;
            r[e] = !kept ? 0.0f
                         : (o.kind == kInfRow ? w_inf : (float)((double)key_mass(key) * inv));
        }
        if constexpr (VEC == 4) {
            ov[iv] = make_float4(r[0], r[1], r[2], r[3]);
        } else {
            ov[iv] = r[0];
        }
    }
}

constexpr int kStatWords = 8;

template <int VEC>
__global__ __launch_bounds__(kBlock) void tes_sample_kernel(
    const float* __restrict__ probs, u32 V, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, u64 seed, u64 offset, int32_t* __restrict__ out_tokens,
    float* __restrict__ renorm, unsigned flags, u32* __restrict__ stats) {
    __shared__ Smem s;
    const u64 t0 = wall_clock64();
    const u32 b = blockIdx.x;
    const float* row = probs + (size_t)b * V;
    const int32_t kin = top_k[b];
    const u32 k_eff = (kin <= 0 || (u32)kin >= V) ? V : (u32)kin;
    const u64 P = fixed_p(top_p[b]);
    const u64 u = philox_uniform(seed, b, offset);
    const bool force_row = flags & TES_FLAG_FORCE_ROW_SELECT;
    const bool tiny = flags & TES_FLAG_TINY_BUFFER;
    const u32 gather_cap = tiny ? 64u : (u32)kCap;

    if (threadIdx.x == 0) {
        s.gctr[0] = s.gctr[1] = s.gctr[2] = 0;
        s.theta = 0;
    }
    Outcome o{};
    bool done = false;
    u64 t1 = t0;
    if (!force_row && k_eff <= kSlabMaxK) {
        __syncthreads();
        const u32 keep_max = tiny ? k_eff : (k_eff > 2048u ? k_eff : 2048u);
        const Fill f = stream_row<VEC, false>(s, row, V, k_eff, keep_max);
        const u32 fill = f.fill;
        o.compactions = f.compactions;
        t1 = wall_clock64();
        o.passes = 1;
        o.path = kPathBuffer;
        // The support is the best k_eff buffered entries.
        const u64 c_k = select_buffer(s, 0, fill, k_eff, false, 0, kNoUpper).c;
        const BufStats st = buffer_stats(s, fill, c_k);
        done = resolve_prefix(s, fill, c_k, st, true, st.mass, P, u, o);
    } else if (!force_row && k_eff == V) {
        for (int i = threadIdx.x; i < kFineBins; i += kBlock) s.hfine[i] = 0;
        __syncthreads();
        const u32 L = tiny ? 64u : kFullKeep;
        const u32 keep_max = tiny ? L : 2048u;
        const Fill f = stream_row<VEC, true>(s, row, V, L, keep_max);
        const u32 fill = f.fill;
        o.compactions = f.compactions;
        t1 = wall_clock64();
        o.passes = 1;
        u64 hm = 0;
        for (int i = threadIdx.x; i < kFineBins; i += kBlock) hm += s.hfine[i];
        const u64 M = block_sum(s, hm);
        const u64 lo = s.theta;
        const BufStats st = buffer_stats(s, fill, lo);
        o.path = kPathHit;
        done = resolve_prefix(s, fill, lo, st, false, M, P, u, o);
        if (!done && st.ninf == 0 && M > 0) {
            o.path = kPathGather;
            done = resolve_gather<VEC>(s, row, V, tiny ? kCap - 64u : fill, M, P, u, o);
        }
    } else {
        __syncthreads();
    }
    if (!done) {
        o.path = kPathRowSelect;
        resolve_row<VEC>(s, row, V, k_eff, P, u, gather_cap, o);
    }
    const u64 t2 = wall_clock64();
    if (threadIdx.x == 0) out_tokens[b] = (int32_t)o.token;
    if (renorm) write_renorm<VEC>(row, renorm + (size_t)b * V, V, o);
    if (stats) {
        __syncthreads();
        if (threadIdx.x == 0) {
            u32* st = stats + (size_t)kStatWords * b;
            st[0] = o.path;
            st[1] = o.passes + (renorm ? 1u : 0u);
            st[2] = o.compactions;
            st[3] = o.kind;
            st[4] = (u32)(t1 - t0);
            st[5] = (u32)(t2 - t1);
            st[6] = (u32)(wall_clock64() - t2);
            st[7] = o.gathered;
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
struct tes_sampler {
    int device;
    int max_batch;
    int max_vocab;
    unsigned flags;
    u32* d_stats;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) {
            ok = false;
            return;
        }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

}  // namespace

extern "C" int sampler_create(tes_sampler** out, int device, int max_batch, int max_vocab,
                              unsigned flags) {
    if (!out) return TES_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    if (max_batch < 1 || max_vocab < 1 || max_vocab > (1 << 30) || device < 0)
        return TES_ERR_INVALID_ARGUMENT;
    if (flags & ~(TES_FLAG_FORCE_ROW_SELECT | TES_FLAG_TINY_BUFFER | TES_FLAG_STATS))
        return TES_ERR_INVALID_ARGUMENT;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return TES_ERR_NO_DEVICE;
    }
    if (device >= n) return TES_ERR_NO_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return TES_ERR_NO_DEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return TES_ERR_UNSUPPORTED_DEVICE;
    tes_sampler* s = new (std::nothrow) tes_sampler{device, max_batch, max_vocab, flags, nullptr};
    if (!s) return TES_ERR_OUT_OF_MEMORY;
    if (flags & TES_FLAG_STATS) {
        DeviceGuard g(device);
        if (!g.ok || hipMalloc(&s->d_stats, sizeof(u32) * kStatWords * (size_t)max_batch) != hipSuccess) {
            delete s;
            return TES_ERR_OUT_OF_MEMORY;
        }
    }
    *out = s;
    return TES_OK;
}

extern "C" int topk_topp_sample(tes_sampler* s, const float* probs, int B, int V,
                                const int32_t* top_k, const float* top_p, uint64_t seed,
                                uint64_t offset, int32_t* out_tokens, float* renorm_out,
                                void* stream) {
    if (!s || B < 0 || V < 1) return TES_ERR_INVALID_ARGUMENT;
    if (B > s->max_batch || V > s->max_vocab) return TES_ERR_TOO_LARGE;
    if (B == 0) return TES_OK;
    if (!probs || !top_k || !top_p || !out_tokens) return TES_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)probs & 3) || ((uintptr_t)top_k & 3) || ((uintptr_t)top_p & 3) ||
        ((uintptr_t)out_tokens & 3) || ((uintptr_t)renorm_out & 3))
        return TES_ERR_INVALID_ARGUMENT;
    const bool vec4 = (V % 4 == 0) && (((uintptr_t)probs & 15) == 0) &&
                      (((uintptr_t)renorm_out & 15) == 0);
    DeviceGuard g(s->device);
    if (!g.ok) return TES_ERR_LAUNCH;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    u32* stats = (s->flags & TES_FLAG_STATS) ? s->d_stats : nullptr;
    if (vec4)
        hipLaunchKernelGGL(tes_sample_kernel<4>, dim3(B), dim3(kBlock), 0, st, probs, (u32)V,
                           top_k, top_p, seed, offset, out_tokens, renorm_out, s->flags, stats);
    else
        hipLaunchKernelGGL(tes_sample_kernel<1>, dim3(B), dim3(kBlock), 0, st, probs, (u32)V,
                           top_k, top_p, seed, offset, out_tokens, renorm_out, s->flags, stats);
    if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
    return TES_OK;
}

extern "C" int sampler_destroy(tes_sampler* s) {
    if (!s) return TES_OK;
    if (s->d_stats) {
        DeviceGuard g(s->device);
        (void)hipFree(s->d_stats);
    }
    delete s;
    return TES_OK;
}

extern "C" const char* sampler_status_string(int status) {
    switch (status) {
        case TES_OK: return "success";
        case TES_ERR_INVALID_ARGUMENT: return "invalid argument (handle, pointer, size or alignment)";
        case TES_ERR_NO_DEVICE: return "no HIP device available at the requested index";
        case TES_ERR_UNSUPPORTED_DEVICE: return "device is not gfx950 (MI355X)";
        case TES_ERR_OUT_OF_MEMORY: return "allocation failed";
        case TES_ERR_LAUNCH: return "HIP runtime error while enqueueing the kernel";
        case TES_ERR_TOO_LARGE: return "batch or vocabulary above the sampler's limits";
        default: return "unknown status";
    }
}

extern "C" int sampler_get_stats(tes_sampler* s, uint32_t* host_out, int B) {
    if (!s || !host_out || B < 0 || B > s->max_batch) return TES_ERR_INVALID_ARGUMENT;
    if (!s->d_stats) return TES_ERR_INVALID_ARGUMENT;
    DeviceGuard g(s->device);
    if (!g.ok) return TES_ERR_LAUNCH;
    if (hipDeviceSynchronize() != hipSuccess) return TES_ERR_LAUNCH;
    if (hipMemcpy(host_out, s->d_stats, sizeof(u32) * kStatWords * (size_t)B, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return TES_ERR_LAUNCH;
    return TES_OK;
}
