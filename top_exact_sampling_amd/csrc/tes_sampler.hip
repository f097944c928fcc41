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
// Design.
//   * Every entry is a 64-bit composite (key << 32) | ~index, key = the
//     sanitised fp32 bits.  Composites are unique and order entries exactly as
//     the stable descending sort does.
//   * One work item per 512-thread workgroup (two per CU), in block order:
//     the segments of the top-p-only rows (k >= V) first, cut into
//     segments of at most 8192 16-byte vectors (held in registers for
//     probability rows, streamed twice for logit rows) and placed
//     consecutively so that a row's segments run at the same time; then
//     whole-row rows, top-k rows and greedy rows, one item each (top-k rows,
//     and greedy rows if there is still room, become two items when every
//     item fits the resident workgroups).  Streamed rows keep sixteen 16-byte
//     loads per thread in flight.
//   * Greedy rows (k = 1): a running maximum of the raw bits as signed
//     integers per vector, then a reload of the vectors holding the maximum
//     for its smallest index.
//   * Top-k rows (k <= 1024): a threshold key from a sampled histogram of the
//     first loads, then every entry at or above it goes to an LDS candidate
//     buffer (per-wave regions, ballot ranks, no atomics).  A binned finish
//     (one table of per-bin counts and masses, single-wave sorts of the few
//     bins the k-th entry, the top-p boundary and the draw fall in) resolves
//     the row.  This stands in for the radix select and candidate list of the
//     cake_sampling page.
//   * Top-p-only rows: each segment builds an exact mass histogram over
//     1/128-octave key bins in LDS.  Two small exchanges follow through a
//     per-row workspace (device-coherent stores, then a relaxed arrival
//     counter; readers acquire; every wait is bounded): the summed 1/8-octave
//     histogram names the coarse bin of the top-p boundary and the coarse bins
//     the draw can fall in, and the fine bins of just those coarse bins then
//     name the fine boundary bin and the fine draw bins (bf16 rows publish
//     their whole fine histograms with the first exchange and skip the
//     second).  Every segment
//     gathers the entries of those few fine bins (from its registers, or a
//     second read of its part for logit rows) and the last segment to arrive
//     finishes with binned selects.  This is the exact-integer analogue of the pivot and
//     sigma-truncation searches of the Qrita paper (sections 3.1-3.2): the
//     boundary is found by mass, never by sorting the nucleus.
//   * Top-p-only rows of launches whose segments would not all be resident
//     at once: one workgroup per row, one pass that bins every entry and
//     appends those of predicted bins, then selects among them.
//   * Rows with 1024 < k < V, and any row whose fast path cannot decide
//     (over-full gather, too many draw bins, an exchange that times out), are
//     resolved by one workgroup with exact multi-pass radix selects over the
//     whole row.
//   * renorm_out is written by a second kernel from the per-row decision
//     (and, for top-k and greedy rows, their recorded kept entries); the
//     slab export sorts each row's support (for top-k and greedy rows, from
//     their recorded support entries).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <cstring>
#include <mutex>
#include <new>
#include <type_traits>

#include "tes_sampler.h"

typedef uint64_t u64;
typedef uint32_t u32;
typedef uint16_t u16;

namespace {

constexpr int kBlock = 512;            // threads per workgroup (8 waves)
constexpr int kWaves = kBlock / 64;
constexpr int kWavesPerSimd = 4;       // two workgroups per CU
constexpr int kSlotsFull = 16;         // vectors per thread of a register-resident segment
constexpr u32 kSegVecFull = kBlock * kSlotsFull;
// Rows of 8-entry (bf16) vectors keep half as many vectors per thread, so that
// a segment holds as many entries as one of fp32 rows.
template <int VEC>
constexpr int kSlots = VEC == 8 ? kSlotsFull / 2 : kSlotsFull;
constexpr u32 kSegVecSmall = kBlock * 2;     // segment size under TES_FLAG_SMALL_SEGMENTS
constexpr u32 kStreamDepth = 16;       // 16-byte loads per thread in flight when streaming
constexpr u32 kPassDepth = 8;          // the same for the passes of whole-row selects
constexpr u32 kGreedyYieldDepth = 2;   // the same for greedy rows that yield bandwidth
constexpr u32 kSampleDepth = 4;        // leading steps of a top-k stream that set its threshold
constexpr u32 kChunk = 1024;           // rows per launch
constexpr u32 kSlabMaxK = 1024;        // largest k served by the streaming top-k path
static_assert(kSlabMaxK < 65536, "top-k row k is kept as u16");
constexpr size_t kWsBudget = 512u << 20;  // workspace bytes per sampler (rows per launch follow)
constexpr int kBins = 2048;            // 11-bit radix digits
constexpr u32 kInfKey = 0x7F800000u;
constexpr u32 kOneKey = 0x3F800000u;   // 1.0f: masses saturate at 2^32 from here
constexpr u32 kMinMassKey = 95u << 23; // 2^-32: the smallest value with a nonzero mass
constexpr int kFineShift = 16;         // fine bins: exponent + 7 mantissa bits
constexpr u32 kFineBase = kMinMassKey >> kFineShift;
constexpr int kFineBins = (int)((kOneKey >> kFineShift) - kFineBase) + 1;  // 4097
constexpr int kCoarseBins = (kFineBins - 1) / 16 + 1;                       // 257
constexpr int kDMax = 48;              // coarse bins whose fine bins are exchanged
constexpr u32 kGSeg = 512;             // gathered entries per top-p-only segment
constexpr u32 kSpinLimit = 1u << 16;   // polls before an exchange gives up
constexpr u32 kMaxSegWs = 64;          // exchange slots per row in the workspace
constexpr u64 kNoUpper = ~0ull;
constexpr int kIntMin = -2147483647 - 1;

static_assert(kFineBins == 4097, "fine bin layout");
static_assert(kCoarseBins == 257, "coarse bin layout");

enum RowKind : u32 { kNormal = 0, kInfRow = 1, kZeroRow = 2 };
enum RowClass : u32 { kClsFull = 0, kClsWhole = 1, kClsSlab = 2, kClsGreedy = 3 };
enum RowPath : u32 {
    kPathSlab = 0, kPathFull = 1, kPathFullFallback = 2, kPathWhole = 3, kPathGreedy = 4,
    kPathSlabFallback = 5, kPathFullRow = 6
};
enum RowFlag : u32 { kFlagFail = 1u };
constexpr int kStatWords = 16;  // per-row debug statistics (TES_FLAG_STATS)

// ---------------------------------------------------------------------------
// Workspace layout (device memory owned by the sampler handle)
// ---------------------------------------------------------------------------
struct RowState {  // zero between calls
    u32 arrive_a;  // top-p-only: first exchange
    u32 arrive_b;  // top-p-only: second exchange (fp32 rows)
    u32 ticket;    // last-arriver ticket
    u32 flags;     // kFlagFail
    u32 vticket;   // speculative verification: last-arriver ticket of a request's chunks
    u32 pad[11];
};
static_assert(sizeof(RowState) == 64, "row state size");

// Logit rows: the row maximum, as partial maxima of up to kXParts parts of the
// row written by the prologue kernel (order-preserving u32 encodings).
constexpr u32 kXParts = 8;
struct XMax {
    u32 part[kXParts];
};

struct Decision {  // what renorm_out and the slab export need
    u32 kind;
    u32 m;
    u32 token;
    u32 path;
    u64 c_keep;  // kept entries have composite >= c_keep
    u64 M_p;     // kept mass (normal rows)
    u64 c_k;     // the support is the entries with composite >= c_k (k_eff < V)
    u32 nlist;   // with a row list: its entries, or kNoList
    u32 pad;
};

struct PubC {  // first exchange of a top-p-only segment (and its gather count)
    u64 M;
    u64 ninf;
    u64 ng;      // entries gathered for the final selects (written last)
    u64 mf;      // logit rows with a min-p floor: mass of the entries at or above it
    u64 coarse[kCoarseBins];
};
struct PubF {  // second exchange: fine bins of the listed coarse bins
    u64 fine[kDMax][16];
};

struct Params {
    const float* probs;  // first row of this launch (probabilities, or logits)
    const int32_t* top_k;
    const float* top_p;
    const float* temperature;  // logit rows: per-row temperature, or null (1)
    const float* min_p;        // per-row min-p floor, or null (off)
    int32_t* out_tokens;
    u32* stats;          // per row, 8 words, or null
    unsigned char* ws;
    u64 seed;
    u64 offset;
    u32 V;
    u32 nvec;       // vectors per row
    u32 rows;       // rows in this launch
    u32 row_base;   // global index of the first row (Philox counter, stats)
    u32 seg_vec_full;  // vectors per register-resident segment of a top-p-only row
    u32 s_ws;       // segment slots per row in the workspace
    u32 rowbytes;   // bytes of the per-row exchange area
    u32 chunk;      // rows the workspace holds
    u32 flags;
    u32 split;      // parts a top-k or greedy row may be split into (1 .. kMaxSplit)
    u32 slots;      // workgroups resident at once on the device
    u32 xparts;     // logit rows: partial maxima per row
};

__device__ __forceinline__ RowState* ws_state(const Params& p, u32 r) {
    return reinterpret_cast<RowState*>(p.ws) + r;
}
__device__ __forceinline__ Decision* ws_decision(const Params& p, u32 r) {
    return reinterpret_cast<Decision*>(p.ws + (size_t)p.chunk * sizeof(RowState)) + r;
}
__device__ __forceinline__ XMax* ws_xmax(const Params& p, u32 r) {
    return reinterpret_cast<XMax*>(p.ws + (size_t)p.chunk * (sizeof(RowState) + sizeof(Decision))) + r;
}
__device__ __forceinline__ unsigned char* ws_row(const Params& p, u32 r) {
    return p.ws + (size_t)p.chunk * (sizeof(RowState) + sizeof(Decision) + sizeof(XMax)) +
           (size_t)r * p.rowbytes;
}
__device__ __forceinline__ PubC* pub_c(const Params& p, u32 r, u32 seg) {
    return reinterpret_cast<PubC*>(ws_row(p, r)) + seg;
}
__device__ __forceinline__ PubF* pub_f(const Params& p, u32 r, u32 seg) {
    return reinterpret_cast<PubF*>(ws_row(p, r) + (size_t)p.s_ws * sizeof(PubC)) + seg;
}
__device__ __forceinline__ u64* gather_area(const Params& p, u32 r, u32 seg) {
    return reinterpret_cast<u64*>(ws_row(p, r) + (size_t)p.s_ws * (sizeof(PubC) + sizeof(PubF))) +
           (size_t)seg * kGSeg;
}
// bf16 rows publish a segment's whole fine histogram with the first exchange,
// so that no second exchange is needed.  These areas follow the last row's
// exchange area (s_ws per row), which keeps the other rows' layout as it is.
struct PubFF {
    u64 fine[kFineBins];
};
__device__ __forceinline__ PubFF* pub_ff(const Params& p, u32 r, u32 seg) {
    return reinterpret_cast<PubFF*>(ws_row(p, p.chunk)) + (size_t)r * p.s_ws + seg;
}
// A top-k or greedy row streamed by S <= kMaxSplit workgroups, one part each:
// each publishes its part's result in the row's exchange area, and the last
// to arrive finishes.
struct HalfPub {
    u64 best;  // greedy: the part's largest composite
    u32 fill;  // top-k: candidates the part kept (more than kHalfCap: too many)
    u32 tkey;  // top-k: the part's threshold key
    u32 over;  // top-k: the part cannot be used
    u32 pad[3];
};
constexpr u32 kMaxSplit = 8;     // parts a row may be split into
constexpr u32 kMinPartVec = kStreamDepth * kBlock;  // smallest part: one full burst of loads
constexpr u32 kHalfCap = 2048;   // published candidates per part
constexpr size_t kPartBytes = sizeof(HalfPub) + (size_t)kHalfCap * sizeof(u64);
constexpr size_t kSplitBytes = kMaxSplit * kPartBytes;
__device__ __forceinline__ HalfPub* half_pub(const Params& p, u32 r, u32 h) {
    return reinterpret_cast<HalfPub*>(ws_row(p, r)) + h;
}
__device__ __forceinline__ u64* half_cands(const Params& p, u32 r, u32 h) {
    return reinterpret_cast<u64*>(ws_row(p, r) + kMaxSplit * sizeof(HalfPub)) +
           (size_t)h * kHalfCap;
}
// Pointers to device memory reach the kernel through LDS (see params_from),
// which hides their address space; every access to rows and workspace goes
// through these casts so that it is a global-memory instruction.  (A generic
// "flat" access also counts against the LDS counter, so any LDS wait would
// drain the loads in flight.)
#define TES_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ TES_GLOBAL T* gp(T* a) {
    return (TES_GLOBAL T*)a;
}
template <typename T>
__device__ __forceinline__ T ld_g(const T* a) {
    return *(const TES_GLOBAL T*)a;
}

// Device-coherent accessors for exchanged words.
template <typename T>
__device__ __forceinline__ void st_dev(T* a, T v) {
    __hip_atomic_store(gp(a), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(T* a) {
    return __hip_atomic_load(gp(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T add_dev(T* a, T v) {
    return __hip_atomic_fetch_add(gp(a), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void or_dev(T* a, T v) {
    __hip_atomic_fetch_or(gp(a), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Shared memory
// ---------------------------------------------------------------------------
// LDS regions are shared by phases that never overlap in time:
//   selects     sbuf = entries [0, 16 KiB) (kSelCap), shcnt [16, 24 KiB), shmass [24, 40 KiB)
//   sorting     [0, 32 KiB) as u64[4096] (two halves of up to 2048 entries)
//   top-k rows  candidate buffer [0, 32 KiB) (kSlabCap), digit counts [32, 40 KiB)
//   top-p rows  fine mass histogram [0, 32.8 KiB)
//   bin tables  shtab [32, 48 KiB): 2048 packed (count, mass) words of the binned selects
constexpr u32 kSelCap = 2048;   // entries a select or a sort handles
constexpr u32 kSlabCap = 4096;  // top-k candidate buffer
constexpr int kRegionBytes = 48 * 1024;

struct Smem {
    Params p;                  // this launch's parameters (copied from the kernel arguments)
    // Discard slots of the fine mass histograms, one per lane (slot -1 - lane
    // of shfine; slot -1 is the region's first word): entries below the
    // lowest bin (zeros) are added there, so a row of mostly zeros does not
    // send every lane's atomic to one address.  Never read.
    alignas(16) u64 discard[64];
    unsigned char region[kRegionBytes];
    u64 coarse[kCoarseBins];   // summed coarse masses of a top-p-only row
    u64 csum[3];               // summed mass, +inf count and min-p mass of a top-p-only row
    u64 loc_above[4];          // results of the bin lookups (coarse and fine plans, fine_locate)
    int loc_bin[4];
    u32 gn[kMaxSegWs];         // entries each segment of a top-p-only row gathered
    u64 cabove[kCoarseBins];   // mass of the coarse bins above each bin
    u64 finem[kDMax * 16];     // summed fine masses of the listed coarse bins
    int flist[kDMax];          // listed coarse bins
    u16 rows[kChunk];          // rows of this launch in class order
    u16 slab_k[kChunk];        // k of each top-k row (read with the classes)
    u64 wpart[kWaves];
    u64 bc[4];
    u32 ctr[4];
    u32 misc[8];
    alignas(16) u16 wcnt[2][kWaves];  // per-wave append counts of a streaming step (double-buffered)
    u32 npass;                 // passes over the row of the current item (statistics)
};
static_assert((kFineBins + 1) * 8 <= kRegionBytes, "fine histogram fits the region");
static_assert(offsetof(Smem, region) == offsetof(Smem, discard) + sizeof(u64) * 64 &&
                  offsetof(Smem, region) % 16 == 0,
              "the discard slots sit just below the fine histogram's slot -1");

__device__ __forceinline__ u64* sbuf(Smem& s) { return reinterpret_cast<u64*>(s.region); }
__device__ __forceinline__ u32* shcnt(Smem& s) { return reinterpret_cast<u32*>(s.region + 16384); }
__device__ __forceinline__ u64* shmass(Smem& s) { return reinterpret_cast<u64*>(s.region + 24576); }
// Fine mass histogram of a top-p-only segment: bins [0, kFineBins) plus a
// discard slot at index -1.
__device__ __forceinline__ u64* shfine(Smem& s) { return reinterpret_cast<u64*>(s.region + 8); }
__device__ __forceinline__ u32* shdig(Smem& s) { return reinterpret_cast<u32*>(s.region + 32768); }
__device__ __forceinline__ u64* shtab(Smem& s) { return reinterpret_cast<u64*>(s.region + 32768); }

struct Sel {
    u64 c;      // selected composite
    u64 above;  // weight of the considered entries strictly above it
};

struct Digit {
    u32 d;
    u32 cnt;
    u64 above;
};

struct Outcome {  // a resolved row
    u32 token;
    u32 kind;
    u64 c_keep;  // kept entries have composite >= c_keep
    u64 M_p;     // kept mass (normal rows)
    u32 m;       // kept +inf entries (+inf rows)
    u64 c_k;     // smallest composite of the support (0: the whole row)
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
__device__ __forceinline__ u32 comp_key(u64 c) { return (u32)(c >> 32); }

// floor(min(x, 1) * 2^32) for the non-negative float whose bits are `key`.
// x * 2^32 is exact in fp32 and the conversion truncates, i.e. floors.
__device__ __forceinline__ u64 key_mass(u32 key) {
    if (key >= kOneKey) return 1ull << 32;
    return (u64)(u32)(__uint_as_float(key) * 4294967296.0f);
}

// Adds the raw bits b of an entry to an exact fine mass histogram, branch
// free: the bin (b >> 16) - base is clamped to [dslot, kFineBins - 1] by one
// three-way median, sending keys below 2^-32 to the lane's discard slot
// dslot (< 0: a word of its own, so that rows of mostly zeros do not send
// every lane's atomic to one address) and keys >= 1.0, +inf, NaN and
// negative bits to the top bin; the mass
// floor(x * 2^32) comes from the hardware conversion, which saturates: zero
// for NaN and negatives, exact below 1.0, 2^32 - 1 (kTopUnit) from 1.0 up.
// The top bin thus ends holding kTopUnit times its count, whose mass is
// count * 2^32.
constexpr u64 kTopUnit = 0xFFFFFFFFull;
__device__ __forceinline__ void fine_hist_add(u64* fine, u32 b, int dslot) {
    int bin;
    asm("v_med3_i32 %0, %1, %2, %3"
        : "=v"(bin)
        : "v"((int)(b >> kFineShift) - (int)kFineBase), "v"(dslot), "s"(kFineBins - 1));
    u32 q;
    asm("v_cvt_u32_f32 %0, %1" : "=v"(q) : "v"(__uint_as_float(b) * 4294967296.0f));
    atomicAdd((unsigned long long*)&fine[bin], (unsigned long long)q);
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

// Min-p (SonicSampler paper, appendix C.2, eq. (11), on the fixed-point
// masses): the support keeps entries with q >= theta * q_max.  For theta in
// (0, 1] the floor ceil(theta * q_max) is exact: theta = m * 2^-sh with an
// integer m < 2^24, and q_max <= 2^32, so m * q_max fits 64 bits.  NaN and
// theta <= 0 give 0 (off); theta > 1 counts as 1.
__device__ __forceinline__ u64 minp_floor(float theta, u64 qmax) {
    if (!(theta > 0.0f)) return 0;
    const u32 b = __float_as_uint(theta >= 1.0f ? 1.0f : theta);
    const u32 ex = b >> 23;
    const u64 m = ex ? (u64)((b & 0x7FFFFFu) | 0x800000u) : (u64)(b & 0x7FFFFFu);
    const int sh = 150 - (int)(ex ? ex : 1u);  // theta = m * 2^-sh
    const u64 prod = m * qmax;
    if (sh >= 64) return prod != 0 ? 1 : 0;
    return (prod >> sh) + ((prod & ((1ull << sh) - 1)) != 0);
}

// The smallest key whose mass floor(x * 2^32) is at least F (F <= 2^32): the
// bits of the smallest float >= F * 2^-32.
__device__ __forceinline__ u32 minp_key(u64 F) {
    if (F == 0) return 0;
    if (F >= (1ull << 32)) return kOneKey;
    float f = (float)F;                               // nearest
    if ((double)f < (double)F) f = __uint_as_float(__float_as_uint(f) + 1u);  // round up
    return __float_as_uint(f * 0x1p-32f);             // exact scaling (F >= 1)
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): key (seed lo, seed hi),
// counter (offset lo, offset hi, row lo, row hi).  A row's own draw uses
// word0 | word1 << 32 (philox_uniform); the acceptance test of speculative
// verification uses word2 | word3 << 32 of the same block (HI).
template <bool HI = false>
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
    return HI ? ((u64)x2 | ((u64)x3 << 32)) : ((u64)x0 | ((u64)x1 << 32));
}

// ---------------------------------------------------------------------------
// Wave / block primitives (wave64, 8 waves)
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32 lane_id() { return threadIdx.x & 63u; }
__device__ __forceinline__ u32 wave_id() { return threadIdx.x >> 6; }

// Values every lane holds identically (read from LDS or derived from such);
// moving them to scalar registers keeps vector registers for row data.
__device__ __forceinline__ u32 uni(u32 v) { return (u32)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ u64 uni(u64 v) {
    return ((u64)uni((u32)(v >> 32)) << 32) | (u64)uni((u32)v);
}

// The launch parameters, read from LDS into scalar registers.
__device__ __forceinline__ Params params_from(const Smem& s) {
    Params p;
    p.probs = reinterpret_cast<const float*>(uni((u64)s.p.probs));
    p.top_k = reinterpret_cast<const int32_t*>(uni((u64)s.p.top_k));
    p.top_p = reinterpret_cast<const float*>(uni((u64)s.p.top_p));
    p.temperature = reinterpret_cast<const float*>(uni((u64)s.p.temperature));
    p.min_p = reinterpret_cast<const float*>(uni((u64)s.p.min_p));
    p.out_tokens = reinterpret_cast<int32_t*>(uni((u64)s.p.out_tokens));
    p.stats = reinterpret_cast<u32*>(uni((u64)s.p.stats));
    p.ws = reinterpret_cast<unsigned char*>(uni((u64)s.p.ws));
    p.seed = uni(s.p.seed);
    p.offset = uni(s.p.offset);
    p.V = uni(s.p.V);
    p.nvec = uni(s.p.nvec);
    p.rows = uni(s.p.rows);
    p.row_base = uni(s.p.row_base);
    p.seg_vec_full = uni(s.p.seg_vec_full);
    p.s_ws = uni(s.p.s_ws);
    p.rowbytes = uni(s.p.rowbytes);
    p.chunk = uni(s.p.chunk);
    p.flags = uni(s.p.flags);
    p.split = uni(s.p.split);
    p.slots = uni(s.p.slots);
    p.xparts = uni(s.p.xparts);
    return p;
}

__device__ __forceinline__ u32 mbcnt64(u64 m) {
    return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, 0u));
}

// The value lane (l ^ m) holds, for m = 1, 2, 4, 8, 16 or 32, without going
// through LDS: DPP quad permutes and (half-)row mirrors compose to the xors
// within 16 lanes (xor 4 = quad reverse then half-row mirror, xor 8 =
// half-row mirror then row mirror), ds_swizzle in bit mode gives xor 16 and
// permlane32_swap exchanges the two halves of the wave.
__device__ __forceinline__ u32 lane_xor(u32 v, u32 m) {
    const int x = (int)v;
    switch (m) {
        case 1: return (u32)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
        case 2: return (u32)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
        case 4:
            return (u32)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false),
                                                 0x141, 0xF, 0xF, false);
        case 8:
            return (u32)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false),
                                                 0x140, 0xF, 0xF, false);
        case 16: return (u32)__builtin_amdgcn_ds_swizzle(x, 0x401F);
        default: {
            const auto pr = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            return threadIdx.x & 32u ? pr[0] : pr[1];
        }
    }
}
__device__ __forceinline__ u64 lane_xor64(u64 v, u32 m) {
    return ((u64)lane_xor((u32)(v >> 32), m) << 32) | (u64)lane_xor((u32)v, m);
}

__device__ __forceinline__ u64 wave_sum(u64 v) {
#pragma unroll
    for (u32 o = 32; o >= 1; o >>= 1) v += lane_xor64(v, o);
    return v;
}
__device__ __forceinline__ u64 wave_min(u64 v) {
#pragma unroll
    for (u32 o = 32; o >= 1; o >>= 1) {
        const u64 w = lane_xor64(v, o);
        v = w < v ? w : v;
    }
    return v;
}
__device__ __forceinline__ u64 wave_max(u64 v) {
#pragma unroll
    for (u32 o = 32; o >= 1; o >>= 1) {
        const u64 w = lane_xor64(v, o);
        v = w > v ? w : v;
    }
    return v;
}

__device__ __forceinline__ u64 read_lane(u64 v, u32 lane) {
    return ((u64)(u32)__builtin_amdgcn_readlane((int)(u32)(v >> 32), (int)lane) << 32) |
           (u64)(u32)__builtin_amdgcn_readlane((int)(u32)v, (int)lane);
}

// The value of the lane CTRL (a DPP row shift) names, 0 where that lane lies
// outside the row of 16.
template <int CTRL>
__device__ __forceinline__ u64 dpp_shift64(u64 v) {
    const u32 lo = (u32)__builtin_amdgcn_update_dpp(0, (int)(u32)v, CTRL, 0xF, 0xF, true);
    const u32 hi = (u32)__builtin_amdgcn_update_dpp(0, (int)(u32)(v >> 32), CTRL, 0xF, 0xF, true);
    return ((u64)hi << 32) | lo;
}

// Inclusive prefix sum across the wave (all lanes active): shifts by 1, 2, 4
// and 8 within each row of 16 lanes, then the totals of the rows below.
__device__ __forceinline__ u64 wave_incl_scan(u64 x) {
    x += dpp_shift64<0x111>(x);  // row_shr:1
    x += dpp_shift64<0x112>(x);  // row_shr:2
    x += dpp_shift64<0x114>(x);  // row_shr:4
    x += dpp_shift64<0x118>(x);  // row_shr:8
    const u64 r0 = read_lane(x, 15), r1 = read_lane(x, 31), r2 = read_lane(x, 47);
    const u32 lane = lane_id();
    const u64 off = lane < 16u ? 0ull : lane < 32u ? r0 : lane < 48u ? r0 + r1 : r0 + r1 + r2;
    return x + off;
}

// Sum over the workgroup, through kWaves words of LDS at part.
__device__ u64 block_sum_u64(u64* part, u64 v) {
    v = wave_sum(v);
    if (lane_id() == 0) part[wave_id()] = v;
    __syncthreads();
    u64 t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += part[w];
    __syncthreads();
    return uni(t);
}
__device__ u64 block_sum(Smem& s, u64 v) { return block_sum_u64(s.wpart, v); }
__device__ u64 block_min(Smem& s, u64 v) {
    v = wave_min(v);
    if (lane_id() == 0) s.wpart[wave_id()] = v;
    __syncthreads();
    u64 t = ~0ull;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t = s.wpart[w] < t ? s.wpart[w] : t;
    __syncthreads();
    return uni(t);
}
__device__ u64 block_max(Smem& s, u64 v) {
    v = wave_max(v);
    if (lane_id() == 0) s.wpart[wave_id()] = v;
    __syncthreads();
    u64 t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t = s.wpart[w] > t ? s.wpart[w] : t;
    __syncthreads();
    return uni(t);
}

// Exclusive prefix sum over the workgroup in thread order, through kWaves
// words of LDS at part.
__device__ __forceinline__ u64 block_excl_scan_u64(u64* part, u64 v) {
    const u64 x = wave_incl_scan(v);
    const u32 lane = lane_id();
    if (lane == 63) part[wave_id()] = x;
    __syncthreads();
    u64 pre = 0;
    const u32 w0 = wave_id();
    for (u32 w = 0; w < w0; ++w) pre += part[w];
    __syncthreads();
    return pre + x - v;
}
__device__ __forceinline__ u64 block_excl_scan(Smem& s, u64 v) {
    return block_excl_scan_u64(s.wpart, v);
}

// Append `c` at arr[base + slot] for every lane with pred set; slots come from
// one LDS atomic per wave on *ctr.  Slots at or beyond `cap` are counted but
// not written.  Must be reached by whole waves.
__device__ __forceinline__ void wave_append(u64* arr, bool pred, u64 c, u32* ctr, u32 base,
                                            u32 cap) {
    const u64 m = __ballot(pred);
    if (m == 0) return;
    const int leader = __ffsll((unsigned long long)m) - 1;
    u32 pos0 = 0;
    if ((int)lane_id() == leader) pos0 = atomicAdd(ctr, (u32)__popcll(m));
    pos0 = __shfl(pos0, leader, 64);
    const u32 pos = base + pos0 + mbcnt64(m);
    if (pred && pos < cap) arr[pos] = c;
}

// Appends, for every lane, its entries c[e] whose bit e is set in `mask`
// (e < N) at arr[base + ...]: slots in lane order from one LDS atomic per wave
// for the wave's total, each lane's offset from a prefix sum over the bits of
// its count.  Slots at or beyond `cap` are counted but not written.  Must be
// reached by whole waves.
template <int N>
__device__ __forceinline__ void wave_append_n(u64* arr, u32 mask, const u64 (&c)[N], u32* ctr,
                                              u32 base, u32 cap) {
    const u32 cnt = (u32)__popc(mask);
    const u64 any = __ballot(cnt != 0);
    if (any == 0) return;
    u32 pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; (1 << b) <= N; ++b) {
        const u64 bb = __ballot((cnt >> b) & 1u);
        pre += mbcnt64(bb) << b;
        tot += (u32)__popcll(bb) << b;
    }
    const int leader = __ffsll((unsigned long long)any) - 1;
    u32 pos0 = 0;
    if ((int)lane_id() == leader) pos0 = atomicAdd(ctr, tot);
    pos0 = (u32)__builtin_amdgcn_readlane((int)pos0, leader);
    u32 pos = base + pos0 + pre;
    // (One condition per store and a branch-free position.)
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const bool take = (mask >> e) & 1u;
        if (take && pos < cap) arr[pos] = c[e];
        pos += take ? 1u : 0u;
    }
}

// Adds word i of every segment's record to acc(i, value) for i < n; record q
// holds u64 words at rec0 + q * stride.  Each thread issues four independent
// loads before using them, so one round trip to L2 serves 2048 words whatever
// the number of segments.
// Sums word i of the nseg published records (record q at rec0 + q * stride)
// for every i < n and hands each sum to acc(i, sum) exactly once.  Each thread
// takes whole words and keeps up to four records' loads in flight.
template <typename Acc>
__device__ __forceinline__ void sum_words(const u64* rec0, u32 stride, u32 nseg, u32 n, Acc acc) {
    for (u32 i = threadIdx.x; i < n; i += kBlock) {
        u64 sum = 0;
        for (u32 q0 = 0; q0 < nseg; q0 += 4) {
            u64 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = q0 + j < nseg ? ld_g(rec0 + (size_t)(q0 + j) * stride + i) : 0ull;
#pragma unroll
            for (int j = 0; j < 4; ++j) sum += v[j];
        }
        acc(i, sum);
    }
}

// Every exchanged word is written with a device-coherent store (st_dev); a
// publication is complete once each wave's stores have completed, which is
// what vm_wait() waits for.  The arrival counters are then bumped with
// relaxed device-scope atomics, and a reader invalidates its caches (acquire)
// after it has seen the count it waits for.
__device__ __forceinline__ void vm_wait() {
    // s_waitcnt vmcnt(0), expcnt and lgkmcnt left unconstrained (gfx9 layout).
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Publish this workgroup's exchanged data and count it in at *ctr.
__device__ void arrive_only(Smem& s, u32* ctr) {
    vm_wait();
    __syncthreads();
    if (threadIdx.x == 0) add_dev(ctr, 1u);
}

// Wait until `n` workgroups have counted in at *ctr (bounded); returns false
// on a timeout.  Under TES_FLAG_NO_WAIT every wait reports a timeout without
// polling, so the timeout path of the callers runs on ordinary inputs.
__device__ bool wait_arrivals(Smem& s, u32* ctr, u32 n) {
    if (threadIdx.x == 0) {
        const bool no_wait = (s.p.flags & TES_FLAG_NO_WAIT) != 0;
        u32 ok = no_wait ? 0u : 1u, it = 0;
        while (!no_wait && ld_dev(ctr) < n) {
            if (++it > kSpinLimit) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s.misc[7] = ok;
    }
    __syncthreads();
    const bool ok = uni(s.misc[7]) != 0;
    __syncthreads();
    return ok;
}

// arrive_only, then wait_arrivals.
__device__ bool arrive_wait(Smem& s, u32* ctr, u32 n) {
    arrive_only(s, ctr);
    return wait_arrivals(s, ctr, n);
}

// Count in at the row's ticket; true in the workgroup that arrives last, which
// has then acquired everything the others published.
__device__ bool arrive_last(Smem& s, u32* ticket, u32 n) {
    vm_wait();
    __syncthreads();
    if (threadIdx.x == 0) {
        const u32 t = add_dev(ticket, 1u);
        s.misc[6] = (t == n - 1) ? 1u : 0u;
        if (t == n - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    const bool last = uni(s.misc[6]) != 0;
    __syncthreads();
    return last;
}

// Adds one to hc[d] (and, for mass tables, q to hm[d]) for every lane with
// pred set.  When at least 8 active lanes share the first active lane's digit
// (ties, runs of zeros), those lanes are summed across the wave and added by
// one lane: LDS atomics to one address from many lanes are serialised, which
// made rows of equal values orders of magnitude slower than others.  Must be
// reached by whole waves.
__device__ __forceinline__ void hist_add(u32* hc, u64* hm, bool mass, bool pred, u32 d, u64 q) {
    const u64 act = __ballot(pred);
    if (act == 0) return;
    const int lead = __builtin_ctzll(act);
    const u32 d0 = (u32)__builtin_amdgcn_readlane((int)d, lead);
    const u64 sm = __ballot(pred && d == d0);
    if (__popcll(sm) < 8) {
        if (pred) {
            atomicAdd(&hc[d], 1u);
            if (mass) atomicAdd((unsigned long long*)&hm[d], (unsigned long long)q);
        }
        return;
    }
    const bool same = pred && d == d0;
    if (pred && !same) {
        atomicAdd(&hc[d], 1u);
        if (mass) atomicAdd((unsigned long long*)&hm[d], (unsigned long long)q);
    }
    const u64 qs = mass ? wave_sum(same ? q : 0ull) : 0ull;
    if ((int)lane_id() == lead) {
        atomicAdd(&hc[d0], (u32)__popcll(sm));
        if (mass && qs) atomicAdd((unsigned long long*)&hm[d0], (unsigned long long)qs);
    }
}

// ---------------------------------------------------------------------------
// Histogram search and radix selects
// ---------------------------------------------------------------------------
// Bins [0, nb) taken in descending order: the bin where the cumulative weight
// first reaches W (1 <= W <= total weight); `above` = weight of higher bins,
// `cnt` = count(bin).
template <typename WF, typename CF>
__device__ Digit find_desc(Smem& s, int nb, u64 W, WF weight, CF count) {
    const int per = (nb + kBlock - 1) / kBlock;
    const int top = nb - 1 - (int)threadIdx.x * per;
    u64 local = 0;
    for (int j = 0; j < per; ++j)
        if (top - j >= 0) local += weight(top - j);
    if (threadIdx.x == 0) {
        s.bc[0] = 0;
        s.bc[1] = 0;
        s.bc[3] = 0;
    }
    u64 acc = block_excl_scan(s, local);
    for (int j = 0; j < per; ++j) {
        const int b = top - j;
        if (b >= 0) {
            const u64 w = weight(b);
            if (acc < W && W <= acc + w) {
                s.bc[0] = (u64)b;
                s.bc[1] = acc;
                s.bc[3] = count(b);
            }
            acc += w;
        }
    }
    __syncthreads();
    Digit g;
    g.d = uni((u32)s.bc[0]);
    g.above = uni(s.bc[1]);
    g.cnt = uni((u32)s.bc[3]);
    __syncthreads();
    return g;
}

__device__ __forceinline__ int level_shift(int l) { return l < 5 ? 52 - 11 * l : 0; }
__device__ __forceinline__ int level_width(int l) { return l < 5 ? 11 : 8; }
__device__ __forceinline__ u64 level_high_mask(int l) {
    const int top = level_shift(l) + level_width(l);
    return top >= 64 ? 0ull : (~0ull << top);
}

// Weighted radix select over the entries c given by get(i, c) for i < n with
// lo <= c < hi: the composite at which the descending cumulative weight (one
// per entry, or its mass) first reaches W (1 <= W <= total).  hc (and, for
// mass weights, hm) are LDS digit tables of kBins entries.
template <typename Get>
__device__ Sel radix_select(Smem& s, u32 n, Get get, u64 W, bool mass, u64 lo, u64 hi, u32* hc,
                            u64* hmw) {
    u64 prefix = 0, above = 0;
    for (int l = 0; l < 6; ++l) {
        const int sh = level_shift(l), wd = level_width(l);
        const u64 hm = level_high_mask(l);
        const u32 dmask = (1u << wd) - 1;
        for (int b = threadIdx.x; b < (1 << wd); b += kBlock) {
            hc[b] = 0;
            if (mass) hmw[b] = 0;
        }
        __syncthreads();
        for (u32 i0 = 0; i0 < n; i0 += kBlock) {
            const u32 i = i0 + threadIdx.x;
            u64 c = 0;
            const bool in = i < n && get(i, c) && c >= lo && c < hi && (c & hm) == prefix;
            hist_add(hc, hmw, mass, in, (u32)(c >> sh) & dmask, mass ? key_mass(comp_key(c)) : 0ull);
        }
        __syncthreads();
        auto cf = [&](int b) { return (u64)hc[b]; };
        const Digit g = mass ? find_desc(s, 1 << wd, W - above, [&](int b) { return hmw[b]; }, cf)
                             : find_desc(s, 1 << wd, W - above, cf, cf);
        above += g.above;
        prefix |= (u64)g.d << sh;
        if (g.cnt == 1 || l == 5) {
            const u64 m2 = ~0ull << sh;
            for (u32 i = threadIdx.x; i < n; i += kBlock) {
                u64 c;
                if (get(i, c) && c >= lo && c < hi && (c & m2) == prefix) s.bc[2] = c;
            }
            __syncthreads();
            const Sel r{uni(s.bc[2]), above};
            __syncthreads();
            return r;
        }
    }
    return Sel{0, 0};  // not reached
}

// Select over sbuf(s)[0, n), n <= kSelCap (the digit tables sit above it).
// The finishes are inlined into the kernel: a call boundary makes the caller
// and callee save registers to scratch memory, and reloading them costs a
// memory round trip on every row's critical path (about 1 us per row).
__device__ __forceinline__ Sel select_buf(Smem& s, u32 n, u64 W, bool mass, u64 lo = 0,
                                          u64 hi = kNoUpper) {
    return radix_select(s, n, [&](u32 i, u64& c) { c = sbuf(s)[i]; return true; }, W, mass, lo, hi,
                        shcnt(s), shmass(s));
}

// Count select over the top-k candidate buffer sbuf(s)[0, n), n <= kSlabCap
// (its digit table sits above the buffer).
__device__ __forceinline__ u64 select_slab(Smem& s, u32 n, u64 W) {
    return radix_select(s, n, [&](u32 i, u64& c) { c = sbuf(s)[i]; return true; }, W, false, 0,
                        kNoUpper, shdig(s), nullptr)
        .c;
}

// Keep the entries of sbuf(s)[0, n) (n <= kSlabCap) at or above `keep`, in
// place; returns how many there are.
__device__ __forceinline__ u32 keep_above(Smem& s, u32 n, u64 keep) {
    constexpr int kPer = kSlabCap / kBlock;
    u64 mine[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const u32 i = threadIdx.x + j * kBlock;
        mine[j] = i < n ? sbuf(s)[i] : 0ull;
    }
    u32 mask = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        mask |= (threadIdx.x + j * kBlock < n && mine[j] >= keep) ? 1u << j : 0u;
    if (threadIdx.x == 0) s.ctr[3] = 0;
    __syncthreads();
    wave_append_n<kPer>(sbuf(s), mask, mine, &s.ctr[3], 0, kSlabCap);
    __syncthreads();
    const u32 kept = uni(s.ctr[3]);
    __syncthreads();
    return kept;
}

// ---------------------------------------------------------------------------
// Row data access
// ---------------------------------------------------------------------------
template <int VEC>
struct VecT;
typedef float f4 __attribute__((ext_vector_type(4)));
template <>
struct VecT<4> {
    typedef f4 T;
    __device__ static float get(const T& v, int e) { return v[e]; }
};
template <>
struct VecT<1> {
    typedef float T;
    __device__ static float get(const T& v, int) { return v; }
};
// bf16 rows: eight values per 16-byte vector.  A bf16 value is the upper half
// of an fp32 value with the same bits below zero, so its fp32 widening (the
// bits shifted up by 16) is exact and every rule of the method applies to it
// unchanged.
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
template <>
struct VecT<8> {
    typedef u4v T;
    __device__ static float get(const T& v, int e) {
        return __uint_as_float(((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
    }
};
// Whether any entry of x, its bits read as a signed int, is >= tkey, for a
// tkey that is a multiple of 2^16.  The eight entries of a bf16 vector are
// compared as signed 16-bit halves (packed integer maxima): a widened entry
// (h << 16) >= tkey exactly when the signed half h >= tkey >> 16.
template <int VEC>
__device__ __forceinline__ bool any_at_least(const typename VecT<VEC>::T& x, int tkey) {
    if constexpr (VEC == 8) {
        typedef short s2v __attribute__((ext_vector_type(2)));
        auto halves = [](u32 w) {
            s2v h;
            __builtin_memcpy(&h, &w, sizeof(w));
            return h;
        };
        auto hmax = [](s2v a, s2v b) { return a > b ? a : b; };  // v_pk_max_i16
        const s2v c = hmax(hmax(halves(x.x), halves(x.y)), hmax(halves(x.z), halves(x.w)));
        u32 m;
        __builtin_memcpy(&m, &c, sizeof(m));
        // The upper half compares in place (the lower bits cannot lift it
        // past a multiple of 2^16); the lower half is moved up.
        return max((int)m, (int)(m << 16)) >= tkey;
    } else {
        int mx = (int)__float_as_uint(VecT<VEC>::get(x, 0));
#pragma unroll
        for (int e = 1; e < VEC; ++e) mx = max(mx, (int)__float_as_uint(VecT<VEC>::get(x, e)));
        return mx >= tkey;
    }
}

// Bytes per row entry: 2 for bf16 rows (VEC = 8), else 4.
template <int VEC>
constexpr size_t kEntryBytes = VEC == 8 ? 2 : 4;
// Row r of the [B][V] matrix at `base`.
template <int VEC>
__device__ __forceinline__ const float* row_ptr(const float* base, size_t r, u32 V) {
    return reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(base) +
                                          r * V * kEntryBytes<VEC>);
}

// ---------------------------------------------------------------------------
// Logit rows
// ---------------------------------------------------------------------------
// A logit row is sampled as the row of fp32 weights w = softmax(x / tau)
// scaled so that its largest entry is 1 (SonicSampler appendix C.1: the
// temperature of eq. (8), then the softmax): w = wtop for x == M (the row
// maximum; wtop = 1, or +inf when M = +inf), else E(fl(fl(x - M) * r)) with
// r = fp32(fp64(1 / tau)) (+inf for tau NaN or <= 0, 0 for tau = +inf).  NaN
// logits weigh 0, like -inf; a row whose entries are all -inf or NaN has M set
// to NaN, so every weight is 0.  Every step after that is the probability
// method applied to w (masses floor(w * 2^32); the scale cancels).
//
// E(s) is exp(s) for s <= 0 by a fixed sequence of IEEE-754 fp32 operations:
// Cody and Waite's reduction n = rint(s log2 e), f = s - n ln2 (ln 2 in a high
// and a low part, each step one fused multiply-add), the degree-7 Taylor
// polynomial of exp(f) in Horner form (coefficients the fp32 values nearest
// 1/j!), and the scaling by 2^n.  Results below 2^-125, NaN and s < -104 give
// 0 (nothing subnormal).  Each operation is correctly rounded, so the weights
// are bit-reproducible.
struct RowXf {
    float M;     // row maximum (NaN: every entry masked)
    float r;     // 1 / temperature
    float wtop;  // weight of the entries equal to M
};

__device__ __forceinline__ float exp_weight(float s) {
    const float sc = fmaxf(s, -104.0f);  // NaN -> -104; the result is discarded below
    const float n = rintf(sc * 0x1.715476p+0f);
    float f = __builtin_fmaf(n, -0x1.62e43p-1f, sc);
    f = __builtin_fmaf(n, 0x1.05c61p-29f, f);
    float q = 0x1.a01a02p-13f;
    q = __builtin_fmaf(q, f, 0x1.6c16c2p-10f);
    q = __builtin_fmaf(q, f, 0x1.111112p-7f);
    q = __builtin_fmaf(q, f, 0x1.555556p-5f);
    q = __builtin_fmaf(q, f, 0x1.555556p-3f);
    q = __builtin_fmaf(q, f, 0.5f);
    q = __builtin_fmaf(q, f, 1.0f);
    q = __builtin_fmaf(q, f, 1.0f);
    const float w = __builtin_ldexpf(q, (int)n);
    return (s >= -104.0f && n >= -125.0f) ? w : 0.0f;
}

// Branch free (a per-entry branch costs more than the exponential it skips).
__device__ __forceinline__ float logit_weight(const RowXf& t, float x) {
    const float w = exp_weight((x - t.M) * t.r);
    return x == t.M ? t.wtop : w;
}

// The weights of a loaded vector of a logit row (identity for probability
// rows).  Applied where a vector is consumed, never where its load is issued,
// so that loads stay in flight.
template <int VEC, bool LG>
__device__ __forceinline__ typename VecT<VEC>::T xform(const RowXf& t,
                                                       const typename VecT<VEC>::T& x) {
    if constexpr (!LG) {
        return x;
    } else {
        static_assert(VEC == 4 || VEC == 1, "logit rows are fp32");
        if constexpr (VEC == 4) {
            return f4{logit_weight(t, x[0]), logit_weight(t, x[1]), logit_weight(t, x[2]),
                      logit_weight(t, x[3])};
        } else {
            return logit_weight(t, x);
        }
    }
}

// Row maximum and temperature of logit row r (wave-uniform).
template <bool LG>
__device__ __forceinline__ RowXf row_xf(const Params& p, u32 r) {
    RowXf t{0.0f, 0.0f, 1.0f};
    if constexpr (LG) {
        // The parts' loads issue together (indices past the last part reread it).
        const XMax* xm = ws_xmax(p, r);
        u32 e = 0;
#pragma unroll
        for (u32 i = 0; i < kXParts; ++i) e = max(e, ld_g(&xm->part[min(i, p.xparts - 1)]));
        e = uni(e);
        const u32 bits = (e & 0x80000000u) ? (e & 0x7FFFFFFFu) : ~e;  // order-preserving decode
        const float tau = p.temperature ? ld_g(&p.temperature[r]) : 1.0f;
        t.r = !(tau > 0.0f) ? __uint_as_float(kInfKey) : (float)(1.0 / (double)tau);
        t.M = bits == 0xFF800000u ? __uint_as_float(0x7FC00000u) : __uint_as_float(bits);
        t.wtop = bits == kInfKey ? __uint_as_float(kInfKey) : 1.0f;
        t.M = __uint_as_float(uni(__float_as_uint(t.M)));
        t.r = __uint_as_float(uni(__float_as_uint(t.r)));
        t.wtop = __uint_as_float(uni(__float_as_uint(t.wtop)));
    }
    return t;
}

// Order-preserving u32 encoding of fp32 values (sign bit set for
// non-negative values, all bits inverted for negative ones) and its inverse.
__device__ __forceinline__ u32 ord_enc(float x) {
    const u32 b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord_dec(u32 e) {
    return __uint_as_float((e & 0x80000000u) ? (e & 0x7FFFFFFFu) : ~e);
}

// The smallest logit x <= M (in value order) whose weight's bits are at least
// wkey - 1, for 2 <= wkey <= the bits of the row's top weight.  The fp32
// exponential is monotone up to one ulp (its value never falls more than one
// ulp below its value at any smaller argument, checked over every argument),
// so every logit whose weight reaches wkey is >= this x: the streams test the
// raw logits against it and compute weights only for those that pass.  One
// wave, 64 candidates per round (six rounds for 32 bits); all lanes of the
// wave take part and get the same result.
__device__ __attribute__((always_inline)) float logit_x_threshold(const RowXf& t, u32 wkey) {
    u32 lo = ord_enc(__uint_as_float(0xFF800000u));  // -inf: weight 0, fails
    u32 hi = ord_enc(t.M);                           // M: the top weight, passes
    const u32 lane = lane_id();
    while (hi - lo > 1u) {
        const u32 step = (hi - lo + 63u) / 64u;
        const u32 e = min(lo + (lane + 1u) * step, hi);
        const bool pass = __float_as_uint(logit_weight(t, ord_dec(e))) >= wkey - 1u;
        const u64 m = __ballot(pass) | (1ull << 63);  // lane 63 reaches hi
        const u32 L = (u32)__builtin_ctzll(m);
        const u32 nhi = min(lo + (L + 1u) * step, hi);
        lo = L ? min(lo + L * step, hi) : lo;
        hi = nhi;
    }
    return ord_dec(hi);
}

// Row data is read once: non-temporal loads keep it from displacing the
// exchanged words and the kernel's own code in L2.
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
    return __builtin_nontemporal_load((const TES_GLOBAL T*)p);
}

// Keeps, in place, the composites of each wave's LDS region (wave w's first
// `n` entries at sbuf(s) + w * reg; n is the calling wave's count) whose key
// satisfies pred, and writes the kept entries of all waves, packed, to
// out[0, cap) with device-coherent stores.  Returns how many there are (which
// may exceed cap).
template <typename Pred>
__device__ __forceinline__ u32 filter_regions(Smem& s, u32 reg, u32 n, Pred pred, u64* out,
                                              u32 cap) {
    const u32 wave = uni(wave_id());
    const u32 lane = lane_id();
    u64* const rg = sbuf(s) + wave * reg;
    u32 kept = 0;
    for (u32 j0 = 0; j0 < n; j0 += 64) {
        const bool in = j0 + lane < n;
        const u64 c = in ? rg[j0 + lane] : 0ull;
        const bool keep = in && pred(comp_key(c));
        const u64 m = __builtin_amdgcn_ballot_w64(keep);
        if (keep) rg[kept + mbcnt64(m)] = c;  // never past the entries already read
        kept += (u32)__popcll(m);
    }
    if (lane == 0) s.gn[wave] = kept;
    __syncthreads();
    u32 total = 0, before = 0;
#pragma unroll
    for (u32 w = 0; w < (u32)kWaves; ++w) {
        const u32 cw = uni(s.gn[w]);
        total += cw;
        before += w < wave ? cw : 0u;
    }
    for (u32 j = lane; j < kept; j += 64)
        if (before + j < cap) st_dev(&out[before + j], rg[j]);
    __syncthreads();
    return total;
}

// Collects the composites of this workgroup's entries of a segment whose raw
// bits satisfy pred (which must accept only bits <= those of +inf, i.e. keys
// that sanitising leaves unchanged) and writes the first `cap` (<= kSelCap)
// of them to out[0, cap) with device-coherent stores.  each(f) calls f(x,
// i, in) for every vector x (index i, in: inside the segment) the thread
// holds, the same number of times in every thread.  Each wave first appends
// to its own LDS region of kSelCap / 8 entries (scalar running count plus the
// lane's rank in the element's ballot, no atomics); the regions are then
// packed.  Returns how many there are, which may exceed cap (or be reported
// as cap + 1 when a wave's region overflowed).
template <int VEC, typename Each, typename Pred>
__device__ __forceinline__ u32 gather_seg(Smem& s, Each each, Pred pred, u64* out, u32 cap) {
    typedef typename VecT<VEC>::T VT;
    constexpr u32 kReg = kSelCap / kWaves;
    const u32 wave = uni(wave_id());
    u64* const reg = sbuf(s) + wave * kReg;
    u32 wfill = 0;
    each([&](const VT& x, u32 i, bool in) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const u32 key = __float_as_uint(VecT<VEC>::get(x, e));
            const bool take = in && pred(key);
            const u64 m = __ballot(take);
            if (m) {
                const u32 pos = wfill + mbcnt64(m);
                if (take && pos < kReg) reg[pos] = composite(key, i * VEC + e);
                wfill += (u32)__popcll(m);
            }
        }
    });
    if (lane_id() == 0) s.gn[wave] = wfill;
    __syncthreads();
    u32 total = 0, before = 0;
    bool over = false;
#pragma unroll
    for (u32 w = 0; w < (u32)kWaves; ++w) {
        const u32 cw = uni(s.gn[w]);
        over |= cw > kReg;
        total += cw;
        before += w < wave ? cw : 0u;
    }
    if (over) total = total > cap ? total : cap + 1;  // reported as too many
    // This wave's entries go to out[before, before + n) while below cap.
    const u32 n = wfill < kReg ? wfill : kReg;
    if (!over) {
        for (u32 j = lane_id(); j < n; j += 64)
            if (before + j < cap) st_dev(&out[before + j], reg[j]);
    }
    __syncthreads();
    return total;
}

// Bitonic sort, descending, of buf[0, kBlock * E) (E = 1, 2 or 4; buf holds
// 2 kBlock E words of LDS) by kBlock threads.  Thread t holds positions
// [t * E, t * E + E) in registers: pairs within a thread are exchanged
// directly, pairs within a wave through lane shuffles, and pairs across waves
// through LDS, alternating between the two halves of buf so that each such
// stage needs one barrier.
template <int E, int S>
__device__ __forceinline__ void cas_local(u64 (&v)[E], u32 base, u32 size) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if ((j & S) == 0) {
            const bool desc = ((base + j) & size) == 0;
            const u64 a = v[j], b = v[j + S];
            const bool sw = desc ? (a < b) : (a > b);
            v[j] = sw ? b : a;
            v[j + S] = sw ? a : b;
        }
    }
}

template <int E>
__device__ __forceinline__ void sort_desc_buf(u64* buf, u64 (&v)[E]) {
    constexpr u32 N = kBlock * E;
    const u32 base = threadIdx.x * E;
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = buf[base + j];
    u32 half = 0;
    // Fully unrolled: every stage's kind (in-thread, lane shuffle, LDS) and
    // partner offsets are compile-time constants, and the shuffles of one
    // stage are issued together.
#pragma unroll
    for (u32 size = 2; size <= N; size <<= 1) {
#pragma unroll
        for (u32 stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride < (u32)E) {
                if (stride == 1) {
                    if constexpr (E >= 2) cas_local<E, 1>(v, base, size);
                } else {
                    if constexpr (E >= 4) cas_local<E, 2>(v, base, size);
                }
            } else if (stride < 64u * E) {
                const u32 lo = stride / E;
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const u32 i = base + j;
                    const u64 o = lane_xor64(v[j], lo);
                    const bool keep_max = ((i & stride) == 0) == ((i & size) == 0);
                    v[j] = keep_max ? (o > v[j] ? o : v[j]) : (o < v[j] ? o : v[j]);
                }
            } else {
                u64* bx = buf + half;
                half ^= N;
#pragma unroll
                for (int j = 0; j < E; ++j) bx[base + j] = v[j];
                __syncthreads();
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const u32 i = base + j;
                    const u64 o = bx[i ^ stride];
                    const bool keep_max = ((i & stride) == 0) == ((i & size) == 0);
                    v[j] = keep_max ? (o > v[j] ? o : v[j]) : (o < v[j] ? o : v[j]);
                }
            }
        }
    }
    __syncthreads();
}
template <int E>
__device__ __forceinline__ void sort_desc(Smem& s, u64 (&v)[E]) {
    static_assert(2 * kBlock * E <= kSlabCap, "sort needs two LDS halves");
    sort_desc_buf<E>(sbuf(s), v);
}

// Finish a row from its support sorted descending: positions [0, kk) of the
// register arrays of sort_desc.
template <int E, bool MINP>
__device__ __forceinline__ Outcome resolve_sorted(Smem& s, const u64 (&v)[E], u32 kk, u64 P, u64 u,
                                                  float theta) {
    const u32 base = threadIdx.x * E;
    u64 q[E];
    u64 ninf_l = 0, msum = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const bool in = base + j < kk;
        const u32 key = comp_key(v[j]);
        q[j] = in ? key_mass(key) : 0;
        ninf_l += (in && key == kInfKey) ? 1u : 0u;
        msum += q[j];
    }
#pragma unroll
    for (int j = 0; j < E; ++j)
        if (base + j == kk - 1) s.loc_above[3] = v[j];  // read after block_sum's barriers
    const u64 ninf = block_sum(s, ninf_l);
    Outcome o{};
    const u64 c_k = uni(s.loc_above[3]);
    o.c_k = c_k;
    if (threadIdx.x == 0) s.bc[0] = s.bc[1] = s.bc[2] = s.bc[3] = 0;
    if (ninf > 0) {
        // +inf entries sort first, in index order: keep them all, draw the t-th.
        const u64 t = __umul64hi(u, ninf);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (base + j == t) s.bc[0] = v[j];
            if (base + j == ninf - 1) s.bc[1] = v[j];
        }
        __syncthreads();
        o.kind = kInfRow;
        o.m = (u32)ninf;
        o.token = comp_index(uni(s.bc[0]));
        o.c_keep = uni(s.bc[1]);
        __syncthreads();
        return o;
    }
    const u64 Mk = block_sum(s, msum);
    if (Mk == 0) {
        // No entry of the support has a mass: the smallest index in it.
        u64 mi = ~0ull;
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (base + j < kk) mi = (u64)comp_index(v[j]) < mi ? (u64)comp_index(v[j]) : mi;
        o.kind = kZeroRow;
        o.token = (u32)block_min(s, mi);
        return o;
    }
    u64 T = topp_threshold(P, Mk);
    if (MINP && theta > 0.0f) {
        // Min-p: the positions with q >= the floor are a prefix; the kept set
        // ends where the inclusive mass reaches min(T, their mass).
        u64 qm = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) qm = q[j] > qm ? q[j] : qm;
        const u64 F = minp_floor(theta, block_max(s, qm));
        u64 mf = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) mf += q[j] >= F ? q[j] : 0ull;
        const u64 Mf = block_sum(s, mf);
        T = Mf < T ? Mf : T;
    }
    const u64 ex = block_excl_scan(s, msum);
    u64 acc = ex;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (acc < T && T <= acc + q[j]) {  // the last kept position
            s.bc[0] = acc + q[j];
            s.bc[1] = v[j];
        }
        acc += q[j];
    }
    __syncthreads();
    const u64 M_p = uni(s.bc[0]);
    o.c_keep = uni(s.bc[1]);
    const u64 t = __umul64hi(u, M_p);
    acc = ex;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (acc <= t && t < acc + q[j]) s.bc[2] = v[j];
        acc += q[j];
    }
    __syncthreads();
    o.kind = kNormal;
    o.M_p = M_p;
    o.token = comp_index(uni(s.bc[2]));
    __syncthreads();
    return o;
}

// ---------------------------------------------------------------------------
// Binned selects over a small LDS entry set
// ---------------------------------------------------------------------------
// The entries are counted into 2048 bins that ascend with the composite, a
// descending exclusive scan of the table gives every bin's count and mass
// above it, and the entries are scattered bin by bin.  A position in the
// descending order (by count) or a cumulative mass then names its bin from
// the table alone, and only that bin, at most 64 entries, is sorted, by one
// wave with lane exchanges.  This replaces full sorts and multi-level radix
// selects, whose cost is dominated by workgroup barriers and by the four
// cycles every wave64 ALU instruction occupies a SIMD.
constexpr int kTabBins = 2048;
constexpr int kTabCountShift = 45;  // a bin holds < 2^19 entries of mass <= 2^32 each
constexpr u64 kTabMassMask = (1ull << kTabCountShift) - 1;

// Lanes [0, n) hold entries and lanes above hold zeros (n wave-uniform);
// returns them sorted descending across the wave, by a bitonic network over
// the smallest power of two >= n lanes.
__device__ __forceinline__ u64 wave_sort_desc(u64 v, u32 n) {
    const u32 lane = lane_id();
#pragma unroll
    for (u32 size = 2; size <= 64; size <<= 1) {
        if ((size >> 1) >= n) break;
#pragma unroll
        for (u32 stride = size >> 1; stride > 0; stride >>= 1) {
            const u64 o = lane_xor64(v, stride);
            const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
            v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
        }
    }
    return v;
}

// Bins the entries c[j] with dig[j] >= 0 (J per thread) and scatters them to
// out[] in descending bin order.  Afterwards shtab(s)[b] holds the packed
// count << 45 | mass of the entries in bins above b, the entries of bin b sit,
// in no particular order, at out[count_above(b), count_above(b) + count(b)),
// and the packed total is returned.
template <int J>
__device__ __forceinline__ u64 bin_scatter(Smem& s, const u64 (&c)[J], const int (&dig)[J],
                                           u64* out, bool cleared = false) {
    u64* tab = shtab(s);
    if (!cleared) {  // (a caller that cleared the table earlier has a barrier since)
        for (int b = threadIdx.x; b < kTabBins; b += kBlock) tab[b] = 0;
        __syncthreads();
    }
    u32 slot[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        slot[j] = 0;
        if (dig[j] >= 0) {
            const u64 inc = (1ull << kTabCountShift) | key_mass(comp_key(c[j]));
            slot[j] = (u32)(atomicAdd((unsigned long long*)&tab[dig[j]], (unsigned long long)inc) >>
                            kTabCountShift);
        }
    }
    __syncthreads();
    // Thread t owns bins 2047 - 4t down to 2044 - 4t.
    static_assert(kTabBins == 4 * kBlock, "four bins per thread");
    const int b0 = kTabBins - 1 - 4 * (int)threadIdx.x;
    u64 w[4], loc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[i] = tab[b0 - i];
        loc += w[i];
    }
    u64 ex = block_excl_scan(s, loc);  // its barriers order the reads above before the writes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tab[b0 - i] = ex;
        ex += w[i];
    }
    if (threadIdx.x == kBlock - 1) s.bc[0] = ex;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j)
        if (dig[j] >= 0) out[(u32)(tab[dig[j]] >> kTabCountShift) + slot[j]] = c[j];
    __syncthreads();
    return uni(s.bc[0]);
}

// Wave-level view of a scattered table: locating bins by cumulative mass and
// sorting one bin.  Every member is wave-uniform except the per-lane v / inc.
struct BinView {
    const u64* tab;
    const u64* srt;
    u64 total;
    int cur = -1;   // bin currently held sorted in v
    u32 st = 0;     // its first position
    u64 v = 0;      // its entries, descending, one per lane (zero past the end)
    u64 inc = 0;    // their inclusive prefix masses within the bin

    __device__ u32 cnt_above(int b) const { return (u32)(tab[b] >> kTabCountShift); }
    __device__ u64 mass_above(int b) const { return tab[b] & kTabMassMask; }
    __device__ u32 end_of(int b) const {
        return b > 0 ? cnt_above(b - 1) : (u32)(total >> kTabCountShift);
    }
    // The bin b with mass_above(b) < W <= mass_above(b) + mass(b), for
    // 1 <= W <= total mass: the last position (descending bins) whose mass
    // above is below W, found 32 bins at a time.
    __device__ int find_mass(u64 W) const {
        const u32 lane = lane_id();
        const u64 a = mass_above(kTabBins - 1 - 32 * (int)lane);
        const u64 m1 = __ballot(a < W);
        const int l1 = 63 - __builtin_clzll(m1);
        const int q = 32 * l1 + (int)(lane & 31u);
        const u64 a2 = mass_above(kTabBins - 1 - q);
        const u64 m2 = __ballot(lane < 32u && a2 < W);
        return kTabBins - 1 - (32 * l1 + (63 - __builtin_clzll(m2)));
    }
    // Loads and sorts bin b; false when it holds more than 64 entries.
    __device__ bool load(int b) {
        if (b == cur) return true;
        st = cnt_above(b);
        const u32 n = end_of(b) - st;
        if (n > 64u) return false;
        const u32 lane = lane_id();
        const u64 x = lane < n ? srt[st + lane] : 0ull;
        v = wave_sort_desc(x, n);
        inc = wave_incl_scan(key_mass(comp_key(v)));
        cur = b;
        return true;
    }
};

// One wave: the j-th smallest (0-based) vocabulary index among the entries
// sbuf(s)[st, st + n), whose indices are distinct.  A radix select on the
// index, 8 bits per round from the highest bit in which the indices differ,
// counting into 256 LDS counters at tab (outside the entries).  All 64 lanes
// must take part.
__device__ __noinline__ u32 wave_nth_index(Smem& s, u32* tab, u32 st, u32 n, u32 j) {
    const u32 lane = lane_id();
    u64 lo = ~0ull, hi = 0;
    for (u32 i = lane; i < n; i += 64) {
        const u64 x = comp_index(sbuf(s)[st + i]);
        lo = x < lo ? x : lo;
        hi = x > hi ? x : hi;
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    const u32 diff = (u32)(lo ^ hi);
    int sh = diff ? ((31 - __builtin_clz(diff)) & ~7) : 0;
    u32 prefix = (u32)lo & ~((2u << (sh + 7)) - 1u);  // bits above the first round
    if (sh + 8 >= 32) prefix = 0;
    u32 pmask = sh + 8 >= 32 ? 0u : ~((1u << (sh + 8)) - 1u);
    for (; sh >= 0; sh -= 8) {
        for (u32 b = lane; b < 256u; b += 64) tab[b] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        for (u32 i0 = 0; i0 < n; i0 += 64) {
            const u32 i = i0 + lane;
            const u32 idx = i < n ? comp_index(sbuf(s)[st + i]) : 0u;
            hist_add(tab, nullptr, false, i < n && (idx & pmask) == prefix, (idx >> sh) & 255u, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const u32 c0 = tab[4 * lane], c1 = tab[4 * lane + 1], c2 = tab[4 * lane + 2],
                  c3 = tab[4 * lane + 3];
        const u32 loc = c0 + c1 + c2 + c3;
        const u32 incl = (u32)wave_incl_scan((u64)loc);
        const u32 excl = incl - loc;
        const u64 m = __builtin_amdgcn_ballot_w64(excl <= j && j < incl);
        const int L = m ? (int)__builtin_ctzll(m) : 0;
        u32 jj = j - (u32)__builtin_amdgcn_readlane((int)excl, L);
        const u32 d0 = (u32)__builtin_amdgcn_readlane((int)c0, L);
        const u32 d1 = (u32)__builtin_amdgcn_readlane((int)c1, L);
        const u32 d2 = (u32)__builtin_amdgcn_readlane((int)c2, L);
        u32 d = 4u * (u32)L;
        if (jj >= d0) {
            jj -= d0;
            ++d;
            if (jj >= d1) {
                jj -= d1;
                ++d;
                if (jj >= d2) {
                    jj -= d2;
                    ++d;
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // reads done before the next clear
        prefix |= d << sh;
        pmask |= 255u << sh;
        j = jj;
    }
    return prefix;
}

// Top-k finish from the candidate buffer sbuf(s)[0, n), k <= n <= kSlabCap,
// which holds every entry of the row with key >= tkey (0 < tkey <= 1.0, a
// multiple of 2^16).  Bins are 1/128-octave key ranges counted from tkey (bin
// 2047 takes every key 16 octaves or more above it, +inf included).  The support's k-th entry, the top-p
// boundary and the drawn entry are each located in the table and resolved by
// sorting their bin.  Returns false, with the buffer holding the same entries
// in another order, when a bin it needs holds more than 64 entries or the
// support holds +inf entries or has no mass; the caller then sorts.
template <bool MINP>
__device__ __forceinline__ bool binned_topk(Smem& s, u32 n, u32 k, u32 tkey, u64 P, u64 u,
                                         Outcome& o, u32 wfill, float theta) {
    constexpr int J = kSlabCap / kBlock;
    static_assert(J * 64 == kSlabCap / kWaves, "a wave region is J entries per lane");
    const u32 tbin = tkey >> kFineShift;
    const bool regions = wfill != ~0u;
    u64 c[J];
    int dig[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        // Packed buffer: thread t takes t + 512 j.  Unpacked wave regions (the
        // stream's, table already cleared): lane l takes l + 64 j of its wave's.
        const u32 i = regions ? wave_id() * (kSlabCap / kWaves) + lane_id() + 64u * j
                              : threadIdx.x + (u32)j * kBlock;
        const bool in = regions ? lane_id() + 64u * j < wfill : i < n;
        c[j] = in ? sbuf(s)[i] : 0ull;
        const u32 d = (comp_key(c[j]) >> kFineShift) - tbin;
        dig[j] = in ? (int)(d < (u32)kTabBins ? d : (u32)kTabBins - 1) : -1;
    }
    // Min-p needs the row's largest key (the buffer holds the row's best k).
    u32 kmax = 0;
    if (MINP && theta > 0.0f) {
        u64 km = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) km = comp_key(c[j]) > km ? comp_key(c[j]) : km;
        kmax = (u32)block_max(s, km);
    }
    __syncthreads();  // the scatter overwrites the buffer
    const u64 total = bin_scatter<J>(s, c, dig, sbuf(s), regions);
    if (wave_id() == 0) {
        BinView bv{shtab(s), sbuf(s), total};
        // +inf entries, the largest keys, can only sit in the top bin.
        const u32 ntop = bv.end_of(kTabBins - 1);
        const u32 lane = lane_id();
        const bool has_inf = ntop > 64u || __ballot(lane < ntop && comp_key(sbuf(s)[lane]) == kInfKey);
        const u32 kkey = comp_key(sbuf(s)[k - 1]);
        const u32 kd = (kkey >> kFineShift) - tbin;
        const int bk = (int)(kd < (u32)kTabBins ? kd : (u32)kTabBins - 1);
        // A bin of more than 64 entries (bv.load fails) whose entries all share
        // one key (long runs of equal values) is ordered by index alone: its
        // position j holds the j-th smallest index, found by a radix select on
        // the index, and every entry has the same mass q, so mass positions
        // are quotients.
        auto tie_key = [&](int b, u32& key) {
            const u32 st0 = bv.cnt_above(b), nb = bv.end_of(b) - st0;
            key = comp_key(sbuf(s)[st0]);
            bool same = true;
            for (u32 i = lane; i < nb; i += 64) same = same && comp_key(sbuf(s)[st0 + i]) == key;
            return __ballot(!same) == 0;
        };
        auto nth = [&](int b, u32 j) {
            // The counters: the top-p-only rows' fine-mass array, unused by
            // top-k rows.
            static_assert(sizeof(s.finem) >= 256 * sizeof(u32), "256 counters fit");
            return wave_nth_index(s, reinterpret_cast<u32*>(s.finem), bv.cnt_above(b),
                                  bv.end_of(b) - bv.cnt_above(b), j);
        };
        bool ok = !has_inf;
        u64 Mk = 0, ck = 0;
        u32 key = 0;
        if (ok) {
            if (bv.load(bk)) {
                Mk = bv.mass_above(bk) + read_lane(bv.inc, k - 1 - bv.st);
                ck = read_lane(bv.v, k - 1 - bv.st);
            } else {
                ok = tie_key(bk, key);
                if (ok) {
                    const u32 j = k - 1 - bv.cnt_above(bk);
                    Mk = bv.mass_above(bk) + (u64)(j + 1) * key_mass(key);
                    ck = composite(key, nth(bk, j));
                }
            }
        }
        ok = ok && Mk > 0;
        u64 cT = 0, Mp = 0, cd = 0;
        if (ok) {
            u64 T = topp_threshold(P, Mk);
            // Min-p: entries with key >= kf are a prefix of the support when
            // kf lies above the k-th entry's key; the kept set then ends where
            // the inclusive mass reaches min(T, their mass): the bins above
            // kf's bin and the entries of kf's bin at or above kf.
            const u64 F = MINP ? minp_floor(theta, key_mass(kmax)) : 0ull;
            const u32 kf = minp_key(F);
            if (MINP && F > 1 && kf > comp_key(ck)) {
                const u32 fd = (kf >> kFineShift) - tbin;
                const int bf = (int)(fd < (u32)kTabBins ? fd : (u32)kTabBins - 1);
                const u32 st0 = bv.cnt_above(bf), en = bv.end_of(bf);
                u64 part = 0;
                for (u32 i = st0 + lane; i < en; i += 64) {
                    const u32 kk = comp_key(sbuf(s)[i]);
                    part += kk >= kf ? key_mass(kk) : 0ull;
                }
                const u64 Mf = bv.mass_above(bf) + wave_sum(part);
                T = Mf < T ? Mf : T;
            }
            const int bT = bv.find_mass(T);
            const u64 base = bv.mass_above(bT);
            if (bv.load(bT)) {
                const u64 mT = __ballot(base + bv.inc >= T);
                ok = mT != 0;  // always set for a consistent table
                if (ok) {
                    const u32 L = (u32)__builtin_ctzll(mT);
                    cT = read_lane(bv.v, L);
                    Mp = base + read_lane(bv.inc, L);
                }
            } else {
                ok = tie_key(bT, key) && key_mass(key) > 0;
                if (ok) {
                    const u64 q = key_mass(key);
                    const u32 j = (u32)((T - base + q - 1) / q) - 1;  // first with base + (j+1) q >= T
                    cT = composite(key, nth(bT, j));
                    Mp = base + (u64)(j + 1) * q;
                }
            }
            if (ok) {
                const u64 t = __umul64hi(u, Mp);
                const int bd = bv.find_mass(t + 1);
                const u64 base2 = bv.mass_above(bd);
                if (bv.load(bd)) {
                    const u64 md = __ballot(base2 + bv.inc > t);
                    ok = md != 0;
                    if (ok) cd = read_lane(bv.v, (u32)__builtin_ctzll(md));
                } else {
                    ok = tie_key(bd, key) && key_mass(key) > 0;
                    if (ok) {
                        const u64 q = key_mass(key);
                        cd = composite(key, nth(bd, (u32)((t - base2) / q)));  // first with base2 + (j+1) q > t
                    }
                }
            }
        }
        if (lane_id() == 0) {
            s.misc[5] = ok ? 1u : 0u;
            s.bc[1] = cT;
            s.bc[2] = Mp;
            s.bc[3] = cd;
            s.loc_above[3] = ck;
        }
    }
    __syncthreads();
    const bool ok = uni(s.misc[5]) != 0;
    o = Outcome{};
    o.kind = kNormal;
    o.c_keep = uni(s.bc[1]);
    o.M_p = uni(s.bc[2]);
    o.token = comp_index(uni(s.bc[3]));
    o.c_k = uni(s.loc_above[3]);
    __syncthreads();
    return ok;
}

// Bins whose nf listed entries all share one key rank them by index alone:
// with mass m per entry, the weight W (1 <= W <= nf m) is reached by the j-th
// lowest index, j = ceil(W / m) - 1, and the j entries before it weigh j m.
// True with the entry's composite in s.bc[1] and the weight above it in
// s.bc[2] (the caller reads them, then synchronises); false when the keys
// differ or carry no mass.  The list is sbuf(s)[kSelCap, kSelCap + nf); all
// threads call it.
__device__ __noinline__ bool tie_select(Smem& s, u32 nf, u64 W) {
    const u64* list = sbuf(s) + kSelCap;
    if (wave_id() == 0) {
        const u32 lane = lane_id();
        u64 kmin = ~0ull, kmax = 0;
        for (u32 i = lane; i < (nf < kSelCap ? nf : kSelCap); i += 64) {
            const u64 kk = comp_key(list[i]);
            kmin = kk < kmin ? kk : kmin;
            kmax = kk > kmax ? kk : kmax;
        }
        kmin = wave_min(kmin);
        kmax = wave_max(kmax);
        const u64 m = nf ? key_mass((u32)kmin) : 0ull;
        const bool tie = nf > 0 && nf <= kSelCap && kmin == kmax && m > 0 && W <= (u64)nf * m;
        if (tie) {
            const u32 j = W ? (u32)((W + m - 1) / m - 1) : 0u;
            // The counters: the table area, past the list.
            const u32 idx = wave_nth_index(s, reinterpret_cast<u32*>(shtab(s)), kSelCap, nf, j);
            if (lane == 0) {
                s.bc[1] = composite((u32)kmin, idx);
                s.bc[2] = (u64)j * m;
            }
        }
        if (lane == 0) s.misc[5] = tie ? 1u : 0u;
    }
    __syncthreads();
    const bool tie = uni(s.misc[5]) != 0;
    if (!tie) __syncthreads();
    return tie;
}

// Mass select inside fine bin f (< kFineBins - 1) over sbuf(s)[0, n), n <=
// kSelCap: the entry at which the bin's descending cumulative mass first
// reaches W (1 <= W <= the bin's mass), with the bin's mass above it.  The
// bin's entries are first compacted into a list.  A list whose entries share
// one key is ranked by index (tie_select): for bf16 rows (kTieFirst) before
// anything else when it holds more than 64, for fp32 rows only once the
// attempts below fail.  Up to 64 entries are sorted
// by one wave; up to 256 are split by one wave into 64 sub-bins of 1024 keys
// (an LDS table of packed count and mass, scanned across the lanes) and only
// the sub-bin holding W is sorted.  Larger bins go through the workgroup's
// 2048-bin table (32 keys per bin), and the radix select decides when even
// that bin holds more than 64 entries.
template <bool kTieFirst>
__device__ __forceinline__ Sel fine_select(Smem& s, u32 n, int f, u64 W) {
    const u32 fkey = (u32)(f + (int)kFineBase);
    u64* list = sbuf(s) + kSelCap;
    if (threadIdx.x == 0) s.ctr[2] = 0;
    __syncthreads();
    for (u32 i0 = 0; i0 < n; i0 += kBlock) {
        const u32 i = i0 + threadIdx.x;
        const u64 c = i < n ? sbuf(s)[i] : 0ull;
        wave_append(list, i < n && (comp_key(c) >> kFineShift) == fkey, c, &s.ctr[2], 0, kSelCap);
    }
    __syncthreads();
    const u32 nf = uni(s.ctr[2]);
    // Rows of bf16 entries: every fine bin holds one value, so a bin of more
    // than 64 entries is a tie run, which the attempts below cannot split.
    if (kTieFirst && nf > 64u && tie_select(s, nf, W)) {
        const Sel t{uni(s.bc[1]), uni(s.bc[2])};
        __syncthreads();
        return t;
    }
    bool ok = false;
    if (nf <= 256u) {
        if (wave_id() == 0) {
            const u32 lane = lane_id();
            bool wok = true;
            u64 v = 0, inc = 0, base = 0;
            if (nf <= 64u) {
                const u64 x = lane < nf ? list[lane] : 0ull;
                v = wave_sort_desc(x, nf);
                inc = wave_incl_scan(key_mass(comp_key(v)));
            } else {
                // 64 sub-bins by key bits 15..10; lane l owns sub-bin 63 - l
                // (descending), entries j * 64 + l are the lane's.
                u64* tab = shtab(s);
                tab[lane] = 0;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                u64 c[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32 i = (u32)j * 64u + lane;
                    c[j] = i < nf ? list[i] : 0ull;
                    if (i < nf)
                        atomicAdd((unsigned long long*)&tab[63 - ((comp_key(c[j]) >> 10) & 63u)],
                                  (unsigned long long)key_mass(comp_key(c[j])));
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                const u64 m = tab[lane];
                const u64 mi = wave_incl_scan(m);
                const u64 me = mi - m;  // mass of the sub-bins above lane's
                const u64 sel = __builtin_amdgcn_ballot_w64(me < W && W <= mi);
                wok = sel != 0;
                const u32 L = wok ? (u32)__builtin_ctzll(sel) : 0u;
                const u32 sb = 63u - L;
                base = read_lane(me, L);
                // Collect the sub-bin's entries into lanes (at most 64).
                u32 cnt = 0;
                u64 x = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32 i = (u32)j * 64u + lane;
                    const bool in = i < nf && ((comp_key(c[j]) >> 10) & 63u) == sb;
                    const u64 bm = __builtin_amdgcn_ballot_w64(in);
                    if (in) {
                        const u32 pos = cnt + mbcnt64(bm);
                        if (pos < 64u) tab[64 + pos] = c[j];
                    }
                    cnt += (u32)__popcll(bm);
                }
                wok = wok && cnt <= 64u;
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                x = (wok && lane < cnt) ? tab[64 + lane] : 0ull;
                v = wave_sort_desc(x, cnt);
                inc = wave_incl_scan(key_mass(comp_key(v)));
            }
            const u64 m = wok ? __builtin_amdgcn_ballot_w64(base + inc >= W) : 0;
            wok = wok && m != 0;
            if (lane == 0) s.misc[5] = wok ? 1u : 0u;
            if (wok) {
                const u32 L = (u32)__builtin_ctzll(m);
                const u64 cw = read_lane(v, L);
                const u64 above = base + read_lane(inc, L) - key_mass(comp_key(cw));
                if (lane == 0) {
                    s.bc[1] = cw;
                    s.bc[2] = above;
                }
            }
        }
        __syncthreads();
        ok = uni(s.misc[5]) != 0;
    } else {
        // The workgroup's table over the list: 2048 bins of 32 keys.
        constexpr int J = kSelCap / kBlock;
        u64 c[J];
        int dig[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const u32 i = threadIdx.x + (u32)j * kBlock;
            c[j] = i < nf ? list[i] : 0ull;
            dig[j] = i < nf ? (int)((comp_key(c[j]) >> 5) & (kTabBins - 1)) : -1;
        }
        __syncthreads();  // the scatter rewrites the list
        const u64 total = bin_scatter<J>(s, c, dig, list);
        if (wave_id() == 0) {
            BinView bv{shtab(s), list, total};
            const int b = bv.find_mass(W);
            bool wok = bv.load(b);
            const u64 base = wok ? bv.mass_above(b) : 0;
            const u64 m = wok ? __ballot(base + bv.inc >= W) : 0;
            wok = m != 0;
            if (lane_id() == 0) s.misc[5] = wok ? 1u : 0u;
            if (wok) {
                const u32 L = (u32)__builtin_ctzll(m);
                const u64 cw = read_lane(bv.v, L);
                const u64 above = base + read_lane(bv.inc, L) - key_mass(comp_key(cw));
                if (lane_id() == 0) {
                    s.bc[1] = cw;
                    s.bc[2] = above;
                }
            }
        }
        __syncthreads();
        ok = uni(s.misc[5]) != 0;
    }
    const Sel r{uni(s.bc[1]), uni(s.bc[2])};
    __syncthreads();
    if (ok) return r;
    if (!kTieFirst && tie_select(s, nf, W)) {
        const Sel t{uni(s.bc[1]), uni(s.bc[2])};
        __syncthreads();
        return t;
    }
    return select_buf(s, n, W, true, fine_lo(f), fine_hi(f));
}

// Calls f(x, iv, valid) for every vector x (index iv) of a row, one per thread
// per round; every thread makes the same number of calls (valid is false past
// the end of the row), so f may use wave collectives.  kG rounds of loads are
// kept in flight.  Logit rows (LG) hand f the vector's weights.
template <int VEC, u32 kG, bool LG = false, typename F>
__device__ __forceinline__ void for_each_vec(const float* __restrict__ row, u32 nvec, F f,
                                             const RowXf& xf = RowXf{}) {
    typedef typename VecT<VEC>::T VT;
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row);
    const u32 nr = (nvec + kBlock - 1) / kBlock;
    const u32 last = nvec - 1;
    VT pf[kG];
#pragma unroll
    for (u32 d = 0; d < kG; ++d) {
        pf[d] = ld_stream(&rv[min(d * kBlock + threadIdx.x, last)]);
        __builtin_amdgcn_sched_barrier(0);  // issue in consumption order
    }
    for (u32 r0 = 0; r0 < nr; r0 += kG) {
#pragma unroll
        for (u32 d = 0; d < kG; ++d) {
            const u32 iv = (r0 + d) * kBlock + threadIdx.x;
            f(xform<VEC, LG>(xf, pf[d]), iv, iv < nvec);
            pf[d] = ld_stream(&rv[min((r0 + d + kG) * kBlock + threadIdx.x, last)]);
            // Keep the refill here: hoisted above the other steps it would
            // turn the pipeline into load-all-then-wait.
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Calls f(key, idx, valid) for every element of a row (sanitised key; the
// weight's key for logit rows).
template <int VEC, bool LG = false, u32 kG = kPassDepth, typename F>
__device__ void for_each_entry(const float* __restrict__ row, u32 nvec, F f,
                               const RowXf& xf = RowXf{}) {
    typedef typename VecT<VEC>::T VT;
    for_each_vec<VEC, kG, LG>(row, nvec, [&](const VT& x, u32 iv, bool valid) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            f(sanitize(__float_as_uint(VecT<VEC>::get(x, e))), iv * VEC + e, valid);
    }, xf);
}

// ---------------------------------------------------------------------------
// Whole-row resolution (1024 < k < V, forced, and fallbacks)
// ---------------------------------------------------------------------------
// Weighted radix select over the entries of the row with composite >= lo:
// histogram one digit per pass; once the selected bucket holds at most
// gather_cap (<= kSelCap) entries, gather it into LDS and finish there.
template <int VEC, bool LG>
__device__ Sel select_row(Smem& s, const float* row, u32 nvec, u64 W, bool mass, u64 lo,
                          u32 gather_cap, const RowXf& xf) {
    u64 prefix = 0, above = 0;
    for (int l = 0; l < 6; ++l) {
        const int sh = level_shift(l), wd = level_width(l);
        const u64 hm = level_high_mask(l);
        const u32 dmask = (1u << wd) - 1;
        for (int b = threadIdx.x; b < kBins; b += kBlock) {
            shcnt(s)[b] = 0;
            shmass(s)[b] = 0;
        }
        __syncthreads();
        for_each_entry<VEC, LG>(row, nvec, [&](u32 key, u32 idx, bool valid) {
            const u64 c = composite(key, idx);
            hist_add(shcnt(s), shmass(s), mass, valid && c >= lo && (c & hm) == prefix,
                     (u32)(c >> sh) & dmask, mass ? key_mass(key) : 0ull);
        }, xf);
        if (threadIdx.x == 0) ++s.npass;
        __syncthreads();
        auto cf = [&](int b) { return (u64)shcnt(s)[b]; };
        const Digit g = mass ? find_desc(s, 1 << wd, W - above, [&](int b) { return shmass(s)[b]; }, cf)
                             : find_desc(s, 1 << wd, W - above, cf, cf);
        above += g.above;
        prefix |= (u64)g.d << sh;
        const u64 m2 = ~0ull << sh;
        if (g.cnt <= gather_cap || l == 5) {
            if (threadIdx.x == 0) s.ctr[3] = 0;
            __syncthreads();
            for_each_entry<VEC, LG>(row, nvec, [&](u32 key, u32 idx, bool valid) {
                const u64 c = composite(key, idx);
                wave_append(sbuf(s), valid && c >= lo && (c & m2) == prefix, c, &s.ctr[3], 0,
                            kSelCap);
            }, xf);
            if (threadIdx.x == 0) ++s.npass;
            __syncthreads();
            const u32 n = uni(s.ctr[3]);
            __syncthreads();
            const Sel r = select_buf(s, n < kSelCap ? n : kSelCap, W - above, mass);
            return Sel{r.c, above + r.above};
        }
    }
    return Sel{0, 0};  // not reached
}

template <int VEC, bool LG>
__device__ __noinline__ Outcome resolve_row(Smem& s, const float* row, u32 nvec, u32 V, u32 k_eff,
                                            u64 P, u64 u, u32 gather_cap, const RowXf& xf,
                                            float theta) {
    Outcome o{};
    u64 lo = 0;
    if (k_eff < V) lo = select_row<VEC, LG>(s, row, nvec, k_eff, false, 0, gather_cap, xf).c;
    o.c_k = lo;
    u64 mk = 0, ninf = 0, minidx = ~0ull, kmax = 0;
    for_each_entry<VEC, LG>(row, nvec, [&](u32 key, u32 idx, bool valid) {
        if (valid && composite(key, idx) >= lo) {
            mk += key_mass(key);
            ninf += key == kInfKey;
            minidx = idx < minidx ? idx : minidx;
            if (LG) kmax = key > kmax ? key : kmax;
        }
    }, xf);
    if (threadIdx.x == 0) ++s.npass;
    const u64 M_k = block_sum(s, mk);
    const u64 m = block_sum(s, ninf);
    minidx = block_min(s, minidx);
    if (m > 0) {
        const u64 t = __umul64hi(u, m);
        o.kind = kInfRow;
        o.m = (u32)m;
        o.token = comp_index(select_row<VEC, LG>(s, row, nvec, t + 1, false, 0, gather_cap, xf).c);
        o.c_keep = select_row<VEC, LG>(s, row, nvec, m, false, 0, gather_cap, xf).c;
        return o;
    }
    if (M_k == 0) {
        o.kind = kZeroRow;
        o.token = (u32)minidx;
        return o;
    }
    u64 T = topp_threshold(P, M_k);
    // Min-p: the support's entries with key >= kf (mass >= the floor) are a
    // prefix; the kept set is the shorter of it and the top-p prefix, i.e.
    // the first position whose inclusive mass reaches min(T, their mass).
    // (Only logit launches carry min-p floors.)
    const u64 F = LG ? minp_floor(theta, key_mass((u32)block_max(s, kmax))) : 0ull;
    const u32 kf = minp_key(F);
    if (LG && F > 1 && kf > comp_key(lo)) {
        u64 mf = 0;
        for_each_entry<VEC, LG>(row, nvec, [&](u32 key, u32 idx, bool valid) {
            if (valid && key >= kf) mf += key_mass(key);
        }, xf);
        if (threadIdx.x == 0) ++s.npass;
        const u64 Mf = block_sum(s, mf);
        T = Mf < T ? Mf : T;
    }
    const Sel bt = select_row<VEC, LG>(s, row, nvec, T, true, lo, gather_cap, xf);
    const u64 M_p = bt.above + key_mass(comp_key(bt.c));
    const u64 t = __umul64hi(u, M_p);
    const Sel dr = select_row<VEC, LG>(s, row, nvec, t + 1, true, lo, gather_cap, xf);
    o.kind = kNormal;
    o.c_keep = bt.c;
    o.M_p = M_p;
    o.token = comp_index(dr.c);
    return o;
}

// ---------------------------------------------------------------------------
// Row completion
// ---------------------------------------------------------------------------
// Row lists, recorded only when renorm_out or the slab export is requested:
// a top-k or greedy row, whose support (the entries with composite >= c_k)
// is at hand when it finishes, writes the composites of its kept entries
// (>= c_keep), or, for the slab export, of its positive support entries, in
// no particular order, to the start of its exchange area and their number to
// its Decision.  The renorm kernel then writes the row's kept entries (the
// list's entries >= c_keep) without reading the row again, and the slab
// export sorts a list that holds the whole support instead of re-reading the
// row.  A row without mass records an empty list; other rows (top-p-only
// rows) record kNoList and are re-read.
constexpr u32 kNoList = ~0u;
// Launch flags (beside the sampler's TES_FLAG_* bits, which never use them):
// record row lists; make them support lists.  (Flags rather than another
// parameter word: the parameters sit in LDS ahead of the work regions, whose
// placement the streams' bank conflicts are sensitive to.)
constexpr u32 kFlagList = 0x80000000u;
constexpr u32 kFlagSupport = 0x40000000u;
__device__ __forceinline__ u64* row_list(const Params& p, u32 r) {
    return reinterpret_cast<u64*>(ws_row(p, r));
}
// Writes the entries c[j] >= c_min held by the workgroup's threads to row r's
// list and returns their number (c_min: c_keep, or c_k for a support list).
// Entries below c_min (zero padding included; c_min > 0) are skipped.  All
// threads call it; the exchange area must no longer be read by anyone.
template <int J>
__device__ u32 emit_list(Smem& s, const Params& p, u32 r, const u64 (&c)[J], u64 c_min) {
    u32 cnt = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) cnt += c[j] >= c_min ? 1u : 0u;
    const u64 x = wave_incl_scan((u64)cnt);
    if (lane_id() == 63) s.wpart[wave_id()] = x;
    __syncthreads();
    u64 pre = 0, tot = 0;
    const u32 w0 = wave_id();
#pragma unroll
    for (u32 w = 0; w < (u32)kWaves; ++w) {
        const u64 t = s.wpart[w];
        pre += w < w0 ? t : 0ull;
        tot += t;
    }
    __syncthreads();
    TES_GLOBAL u64* list = gp(row_list(p, r));
    u32 pos = (u32)(pre + x) - cnt;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const bool take = c[j] >= c_min;
        if (take) list[pos] = c[j];
        pos += take ? 1u : 0u;
    }
    return (u32)tot;
}

__device__ void finish_row(Smem& s, const Params& p, u32 r, const Outcome& o, u32 path,
                           u32 gathered, u32 nlist = kNoList) {
    if (threadIdx.x == 0) {
        if (p.out_tokens) *gp(&p.out_tokens[r]) = (int32_t)o.token;
        Decision* d = ws_decision(p, r);
        *gp(&d->kind) = o.kind;
        *gp(&d->m) = o.m;
        *gp(&d->token) = o.token;
        *gp(&d->path) = path;
        *gp(&d->c_keep) = o.c_keep;
        *gp(&d->c_k) = o.c_k;
        *gp(&d->M_p) = o.M_p;
        const u32 nl = o.kind == kZeroRow ? 0u : nlist;
        *gp(&d->nlist) = nl;
        if (p.stats) {
            u32* st = p.stats + kStatWords * (size_t)(p.row_base + r);
            *gp(&st[0]) = path;
            *gp(&st[1]) = o.kind;
            *gp(&st[4]) = gathered;
            *gp(&st[5]) = (u32)wall_clock64();
            if (nlist != kNoList) *gp(&st[10]) = nl;
        }
    }
}

__device__ void stat_start(const Params& p, u32 r, u32 segments) {
    if (p.stats && threadIdx.x == 0) {
        u32* st = p.stats + kStatWords * (size_t)(p.row_base + r);
        *gp(&st[2]) = segments;
        __hip_atomic_fetch_max(gp(&st[6]), 0xFFFFFFFFu - (u32)wall_clock64(), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void stat_add(const Params& p, u32 r, int word, u32 v) {
    if (p.stats && threadIdx.x == 0 && v)
        add_dev(&p.stats[kStatWords * (size_t)(p.row_base + r) + word], v);
}

// Records why a top-p-only row left its fast path (stats word 7).
__device__ __forceinline__ void stat_why(const Params& p, u32 r, u32 bits) {
    if (p.stats && threadIdx.x == 0)
        __hip_atomic_fetch_or(gp(&p.stats[kStatWords * (size_t)(p.row_base + r) + 7]), bits,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Debug phase timer: adds the ticks since `t` to stats word `word` and
// returns the current tick (only with TES_FLAG_STATS).
__device__ __forceinline__ u64 stat_phase(const Params& p, u32 r, int word, u64 t) {
    if (!p.stats) return 0;
    const u64 now = wall_clock64();
    stat_add(p, r, word, (u32)(now - t));
    return now;
}

// ---------------------------------------------------------------------------
// Greedy rows (k = 1)
// ---------------------------------------------------------------------------
template <int VEC, bool LG>
__device__ __attribute__((always_inline)) void do_greedy(Smem& s, u32 r, u32 h, u32 S, bool yield) {
    const Params p = params_from(s);
    typedef typename VecT<VEC>::T VT;
    const RowXf xf = row_xf<LG>(p, r);
    stat_start(p, r, S);
    const u64 tp = p.stats ? wall_clock64() : 0;
    // This workgroup's part: the row, or one of its S parts when split.
    const u32 hv = (p.nvec + S - 1) / S;
    const u32 v0 = h * hv;
    const u32 nv = min(v0 + hv, p.nvec) - v0;
    const float* part =
        reinterpret_cast<const float*>(reinterpret_cast<const VT*>(row_ptr<VEC>(p.probs, r, p.V)) + v0);
    u64 cbest;
    if constexpr (LG) {
        // Logit rows: the largest weight is the top weight (1 at the row
        // maximum, +inf in rows with +inf logits) and the token is the
        // smallest index whose weight equals it.  Those entries are among
        // the logits >= x1; only their weights are computed.  A row with
        // every logit masked (no entry passes) has only zero weights: its
        // smallest index.
        const u32 wtop = __float_as_uint(xf.wtop);
        const float x1 = logit_x_threshold(xf, wtop);
        u64 bidx = ~0ull;
        auto vfind = [&](const VT& x, u32 iv, bool valid) {
            float mx = VecT<VEC>::get(x, 0);
#pragma unroll
            for (int e = 1; e < VEC; ++e) mx = fmaxf(mx, VecT<VEC>::get(x, e));
            if (valid && mx >= x1) {
#pragma unroll
                for (int e = VEC - 1; e >= 0; --e) {
                    const float xv = VecT<VEC>::get(x, e);
                    if (xv >= x1 && __float_as_uint(logit_weight(xf, xv)) == wtop) {
                        const u64 i = (u64)(v0 + iv) * VEC + e;
                        bidx = i < bidx ? i : bidx;
                    }
                }
            }
        };
        if (yield)
            for_each_vec<VEC, kGreedyYieldDepth>(part, nv, vfind);
        else
            for_each_vec<VEC, kStreamDepth>(part, nv, vfind);
        const u64 idx = block_min(s, bidx);
        cbest = idx == ~0ull ? composite(0u, v0 * VEC) : composite(wtop, (u32)idx);
    } else {
        // The largest bits as signed integers: non-negative floats order as their
        // bits, negative ones (which count as zero) lie below all of them and NaN
        // bits above +inf.  Each lane keeps the first of its vectors holding its
        // largest value; the part's smallest index holding the maximum comes from
        // reloading those vectors afterwards.
        int best = kIntMin;
        u32 bvec = 0;
        auto vmax = [&](const VT& x, u32 iv, bool valid) {
            int mx = (int)__float_as_uint(VecT<VEC>::get(x, 0));
#pragma unroll
            for (int e = 1; e < VEC; ++e) mx = max(mx, (int)__float_as_uint(VecT<VEC>::get(x, e)));
            const bool up = valid && mx > best;
            best = up ? mx : best;
            bvec = up ? iv : bvec;
        };
        // A greedy row needs almost no work after its stream, so when it shares
        // the device with rows that do (top-k finishes, top-p exchanges), it
        // keeps only two loads in flight: its share of the bandwidth goes to those
        // rows, which then finish earlier, and it still ends before them.
        if (yield)
            for_each_vec<VEC, kGreedyYieldDepth, LG>(part, nv, vmax, xf);
        else
            for_each_vec<VEC, kStreamDepth, LG>(part, nv, vmax, xf);
        const int K = (int)((u32)block_max(s, (u64)((u32)best ^ 0x80000000u)) ^ 0x80000000u);
        if (K > (int)kInfKey) {
            // NaN bits are the largest: take the exact maximum of the composites.
            u64 b = 0;
            for_each_entry<VEC, LG>(part, nv, [&](u32 key, u32 idx, bool valid) {
                const u64 c = valid ? composite(key, v0 * VEC + idx) : 0ull;
                b = c > b ? c : b;
            }, xf);
            cbest = block_max(s, b);
        } else if (K <= 0) {
            cbest = composite(0u, v0 * VEC);  // every entry counts as zero: the smallest index
        } else {
            u64 idx = ~0ull;
            if (best == K) {
                const VT x = xform<VEC, LG>(xf, ld_g(&reinterpret_cast<const VT*>(part)[bvec]));
#pragma unroll
                for (int e = VEC - 1; e >= 0; --e)
                    if ((int)__float_as_uint(VecT<VEC>::get(x, e)) == K)
                        idx = (u64)(v0 + bvec) * VEC + e;
            }
            cbest = composite((u32)K, (u32)block_min(s, idx));
        }
    }
    if (S > 1) {
        RowState* rs = ws_state(p, r);
        if (threadIdx.x == 0) st_dev(&half_pub(p, r, h)->best, cbest);
        if (!arrive_last(s, &rs->ticket, S)) return;
        const u64 ob = threadIdx.x < S ? ld_g(&half_pub(p, r, threadIdx.x)->best) : 0ull;
        cbest = block_max(s, ob > cbest ? ob : cbest);
        if (threadIdx.x == 0) st_dev(&rs->ticket, 0u);
    }
    stat_phase(p, r, 8, tp);
    Outcome o{};
    const u32 key = comp_key(cbest);
    o.token = comp_index(cbest);
    o.c_keep = cbest;
    o.c_k = cbest;
    o.m = 1;
    o.M_p = key_mass(key);
    o.kind = key == kInfKey ? kInfRow : (o.M_p == 0 ? kZeroRow : kNormal);
    // The kept entry is the token.
    if ((p.flags & kFlagList) && threadIdx.x == 0) *gp(row_list(p, r)) = cbest;
    finish_row(s, p, r, o, kPathGreedy, 0, (p.flags & kFlagList) ? 1u : kNoList);
}

// ---------------------------------------------------------------------------
// Top-k rows (2 <= k <= 1024)
// ---------------------------------------------------------------------------
template <bool MINP>
__device__ __forceinline__ void slab_finish(Smem& s, u32 r, u32 n, u32 k, u32 tkey, u64 P, u64 u,
                                         u32 wfill, u32 path = kPathSlab, u64 c_k = ~0ull);

// The index of the m-th (m >= 1) entry of the row, in index order, whose key
// is zero (NaN, negative, -0.0 or +0.0), read in steps of one vector per
// thread until a step holds it; ~0u when the row has fewer than m.
template <int VEC, bool LG>
__device__ u32 mth_zero_index(Smem& s, const float* __restrict__ row, u32 nvec, u32 m,
                              const RowXf& xf) {
    typedef typename VecT<VEC>::T VT;
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row);
    u32 before = 0;  // zeros in the steps already read (workgroup-uniform)
    for (u32 v0 = 0; v0 < nvec; v0 += kBlock) {
        const u32 iv = v0 + threadIdx.x;
        u32 zmask = 0;
        if (iv < nvec) {
            const VT x = xform<VEC, LG>(xf, ld_g(&rv[iv]));
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                zmask |= sanitize(__float_as_uint(VecT<VEC>::get(x, e))) == 0u ? 1u << e : 0u;
        }
        const u32 c = (u32)__popc(zmask);
        const u32 ex = (u32)block_excl_scan(s, c);
        if (threadIdx.x == kBlock - 1) s.ctr[2] = ex + c;
        if (threadIdx.x == 0) s.misc[4] = ~0u;
        __syncthreads();
        if (c && before + ex < m && m <= before + ex + c) {
            u32 need = m - before - ex, mm = zmask;  // the need-th set bit of the mask
            while (--need) mm &= mm - 1;
            s.misc[4] = iv * VEC + (u32)__builtin_ctz(mm);
        }
        __syncthreads();
        const u32 hit = uni(s.misc[4]);
        before += uni(s.ctr[2]);
        __syncthreads();
        if (hit != ~0u) return hit;
    }
    return ~0u;
}

// A top-k row whose buffer sbuf(s)[0, n) holds every entry of the row with a
// positive key, n < k: the support is those n entries and the k - n
// lowest-indexed zeros, the last of which is its boundary.  The zeros carry
// no mass, so they are never kept or drawn; only a support without mass
// looks at them (its token is the smallest index in it).
template <int VEC, bool LG>
__device__ __noinline__ void slab_short(Smem& s, u32 r, u32 n, u32 k, u64 P, u64 u, u32 path) {
    const Params p = params_from(s);
    const RowXf xf = row_xf<LG>(p, r);
    const float* row = row_ptr<VEC>(p.probs, r, p.V);
    if (n == 0) {
        // No positive key anywhere: the support is indices [0, k), its
        // boundary index k - 1 and its token 0.
        Outcome o{};
        o.kind = kZeroRow;
        o.token = 0;
        o.c_k = composite(0u, k - 1);
        finish_row(s, p, r, o, path, 0);
        return;
    }
    u64 mn = ~0ull, mass = 0, midx = ~0ull;
    for (u32 i = threadIdx.x; i < n; i += kBlock) {
        const u64 c = sbuf(s)[i];
        mn = c < mn ? c : mn;
        mass += key_mass(comp_key(c));
        midx = comp_index(c) < midx ? comp_index(c) : midx;
    }
    mn = block_min(s, mn);
    mass = block_sum(s, mass);
    const u32 zk = mth_zero_index<VEC, LG>(s, row, p.nvec, k - n, xf);
    const u64 c_k = composite(0u, zk);
    if (mass > 0) {
        // The binned finish's base: at most 1.0, so that +inf entries land in
        // its top bin, where it looks for them.
        slab_finish<LG>(s, r, n, n, min(comp_key(mn), kOneKey) & ~0xFFFFu, P, u, ~0u, path, c_k);
        return;
    }
    midx = block_min(s, midx);
    const u32 z = mth_zero_index<VEC, LG>(s, row, p.nvec, 1, xf);
    Outcome o{};
    o.kind = kZeroRow;
    o.token = (u32)(midx < (u64)z ? midx : (u64)z);
    o.c_k = c_k;
    finish_row(s, p, r, o, path, n);
}

// Exact single pass over the whole row for a top-k row (k <= kSlabMaxK) that
// its sampled threshold could not decide: a sample with too few entries with a
// mass, a candidate buffer that overflowed (long runs of equal values at the
// threshold) or a split row whose parts did not join.  Every entry with key
// >= theta0 (theta0 >= 1) is appended to the LDS buffer; whenever the buffer
// could not take one more step, it is cut to the best k so far (a radix select)
// and the threshold rises to one above the k-th key: the row is read in index
// order, so a later entry with that key has a larger index and ranks below all
// k.  The buffer then holds the row's best k among keys >= theta0, or, when
// fewer exist (theta0 = 1), every entry with a positive key.  A support that
// also reaches zero keys takes the lowest-indexed zeros after them: they carry
// no mass, so they are never kept or drawn, and only a support without mass
// looks at them (its token is the smallest index in the support).
template <int VEC, bool LG>
__device__ __noinline__ void slab_restream(Smem& s, u32 r, u32 k, u32 theta0, u64 P, u64 u) {
    const Params p = params_from(s);
    typedef typename VecT<VEC>::T VT;
    const RowXf xf = row_xf<LG>(p, r);
    const float* row = row_ptr<VEC>(p.probs, r, p.V);
    // Entries are appended kSub per thread at a time (an 8-entry vector in
    // two halves), so the buffer keeps room for one more append.
    constexpr int kSub = VEC > 4 ? 4 : VEC;
    constexpr u32 kHigh = kSlabCap - kBlock * kSub;
    static_assert(kHigh >= kSlabMaxK, "a cut always has k entries to keep");
    u32 theta = theta0;  // workgroup-uniform
    bool closed = false;  // the k-th best so far is +inf: nothing later can enter
    u32 cuts = 0;
    if (threadIdx.x == 0) s.ctr[3] = 0;
    __syncthreads();
    for_each_vec<VEC, kPassDepth, LG>(row, p.nvec, [&](const VT& x, u32 iv, bool valid) {
        // After a cut within a step, entries with the k-th key still enter
        // for the rest of the step (another thread's later half may hold a
        // lower index); only at the step's end does the threshold rise above
        // that key.
        bool raise = false;
#pragma unroll
        for (int h0 = 0; h0 < VEC; h0 += kSub) {
            const u32 span = kInfKey - theta;
            // One append per half: the lane's passing entries go to
            // consecutive slots taken by one LDS atomic per wave.
            u64 c[kSub];
            u32 mask = 0;
#pragma unroll
            for (int e = 0; e < kSub; ++e) {
                const u32 b = __float_as_uint(VecT<VEC>::get(x, h0 + e));
                c[e] = composite(b, iv * VEC + h0 + e);
                mask |= (valid && !closed && b - theta <= span) ? 1u << e : 0u;
            }
            wave_append_n<kSub>(sbuf(s), mask, c, &s.ctr[3], 0, kSlabCap);
            __syncthreads();
            const u32 n = uni(s.ctr[3]);
            if (n > kHigh) {
                __syncthreads();  // every thread has read the count
                const u64 ck = select_slab(s, n, k);
                const u32 kept = keep_above(s, n, ck);
                theta = comp_key(ck);
                raise = true;
                ++cuts;
                if (threadIdx.x == 0) s.ctr[3] = kept;
                __syncthreads();
            }
        }
        if (raise) {
            closed = theta == kInfKey;
            theta = closed ? kInfKey : theta + 1;
        }
    }, xf);
    __syncthreads();
    const u32 n = uni(s.ctr[3]);
    __syncthreads();
    stat_add(p, r, 3, cuts);
    if (n < k) {
        // Fewer than k positive keys (theta0 = 1: from a threshold the row
        // has at least k): the buffer holds every one of them.
        slab_short<VEC, LG>(s, r, n, k, P, u, kPathSlabFallback);
        return;
    }
    u64 mn = ~0ull;
    for (u32 i = threadIdx.x; i < n; i += kBlock) mn = sbuf(s)[i] < mn ? sbuf(s)[i] : mn;
    mn = block_min(s, mn);
    // The binned finish's base: at most 1.0, so that +inf entries land in its
    // top bin, where it looks for them.
    slab_finish<LG>(s, r, n, k, min(comp_key(mn), kOneKey) & ~0xFFFFu, P, u, ~0u, kPathSlabFallback);
}

// Streams its part of the row (the whole row, or one of S <= kMaxSplit parts
// when the row is split between S workgroups) once and keeps, in the LDS
// buffer, every entry whose key is at or above a threshold key tkey > 0,
// chosen so that about 1.5 k (2 k for more than two parts) of the row's share
// pass.  The test is one subtraction and one compare on the raw bits:
// sanitize(b) >= tkey exactly when tkey <= b <= the bits of +inf.
//   The first kSampleDepth steps (2048 entries each, the first loads in
//   flight) are a sample: their keys are counted in 1/128-octave bins before
//   anything else happens, and tkey becomes the lower edge of the bin that
//   holds the sample's j-th best, j = ceil(c k n / V) + 12 for n sampled
//   entries and c = 1.5 or 2 (j = k when the sample is the whole row).
//   Then the part is streamed from its start with no barriers and no atomics:
//   each wave appends to its own region of kSlabCap / 8 entries, at its
//   running count (a scalar) plus the lane's rank among the wave's passing
//   lanes (mbcnt of the element's ballot).  Entries beyond a region are
//   counted but not written.
// The buffer then holds exactly the part's entries at or above tkey.  A whole
// row that kept at least k without overflowing holds the row's best k and is
// finished from the wave regions directly.  The parts of a split row publish
// their buffers and thresholds; the last to arrive keeps every part's entries
// at or above T = the largest threshold (every entry of the row at or above T
// is among them), which hold the row's best k when there are at least k of
// them.  Rows that fail these tests (or whose sample holds fewer than j
// entries with a mass) are decided by the compacting restream.
template <int VEC, bool LG>
__device__ __attribute__((always_inline)) void do_slab(Smem& s, u32 r, u32 k, u32 h, u32 S) {
    const Params p = params_from(s);
    typedef typename VecT<VEC>::T VT;
    const RowXf xf = row_xf<LG>(p, r);
    const u32 hv = (p.nvec + S - 1) / S;
    const u32 v0 = h * hv;
    const u32 nvec = min(v0 + hv, p.nvec) - v0;  // vectors of this part
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row_ptr<VEC>(p.probs, r, p.V)) + v0;
    // Issued before the stream so that its latency is hidden.
    const float top_p = ld_g(&p.top_p[r]);
    stat_start(p, r, S);
    const u64 tp = p.stats ? wall_clock64() : 0;
    const u32 nsteps = (nvec + kBlock - 1) / kBlock;
    const u32 last = nvec - 1;
    u32* hist = reinterpret_cast<u32*>(s.region);  // sample counts per fine bin
    for (int b = threadIdx.x; b < kFineBins; b += kBlock) hist[b] = 0;
    // The binned finish's table (disjoint from the sample counts and the
    // candidate buffer) is cleared here, under the barriers that follow.
    for (int b = threadIdx.x; b < kTabBins; b += kBlock) shtab(s)[b] = 0;
    __syncthreads();
    VT pf[kStreamDepth];
#pragma unroll
    for (u32 d = 0; d < kStreamDepth; ++d) {
        pf[d] = ld_stream(&rv[min(d * kBlock + threadIdx.x, last)]);
        __builtin_amdgcn_sched_barrier(0);  // issue in consumption order
    }
    // The partial last step's vector (if any), loaded early.
    const VT tailv = ld_stream(&rv[min((nvec / kBlock) * kBlock + threadIdx.x, last)]);
    __builtin_amdgcn_sched_barrier(0);
    // The sample.
    u32 nmass = 0;
#pragma unroll
    for (u32 d = 0; d < kSampleDepth; ++d) {
        const bool valid = d * kBlock + threadIdx.x < nvec;
        const VT xs = xform<VEC, LG>(xf, pf[d]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const u32 key = sanitize(__float_as_uint(VecT<VEC>::get(xs, e)));
            if (valid && key >= kMinMassKey) {
                atomicAdd(&hist[fine_bin(key)], 1u);
                ++nmass;
            }
        }
    }
    const u32 nsamp = min(kSampleDepth * kBlock, nvec) * VEC;
    // (1.5 k of the row's share for one or two parts, 2 k beyond: the largest
    // of many parts' thresholds must still leave k entries above it.)
    const u64 kmul = S > 2 ? 4 : 3;
    const u32 j = (S == 1 && nsteps <= kSampleDepth)
                      ? k
                      : (u32)((kmul * k * nsamp + 2ull * p.V - 1) / (2ull * p.V)) + 12;
    const u32 tot = (u32)block_sum(s, nmass);  // also orders the histogram
    u32 tkey = 0;
    if (j <= tot) {
        auto cw = [&](int b) { return (u64)hist[b]; };
        const Digit g = find_desc(s, kFineBins, j, cw, cw);
        tkey = (u32)(g.d + kFineBase) << kFineShift;
    }
    __syncthreads();  // the histogram is dead; the buffer takes its place
    const bool no_tkey = tkey == 0;
    // Fewer than j sampled entries have a mass (a row of mostly zeros, or a
    // short row with fewer than k): the part streams every positive key (if
    // they fit, the row's positive entries are then all at hand).
    if (no_tkey) tkey = 1u;
    const u32 span = kInfKey - tkey;
    // Logit rows: the weights at or above tkey belong to logits >= xb.
    float xb = 0.0f;
    if constexpr (LG) xb = logit_x_threshold(xf, tkey);
    u64 tq = stat_phase(p, r, 11, tp);
    constexpr u32 kRegion = kSlabCap / kWaves;
    const u32 wave = uni(wave_id());
    u64* const reg = sbuf(s) + wave * kRegion;
    u32 wfill = 0;  // entries this wave has appended (wave-uniform)
    // Appends this lane's passing entries of one vector.  Passing bits are
    // non-negative as signed integers, so a vector whose largest signed bits
    // are below tkey has none; a wave with no such vector skips the rest.
    // (MASKED: lanes past the end of the part hold a copy of its last vector
    // and must append nothing.)
    auto append = [&](auto masked, const VT& x, u32 iv) {
        constexpr bool kMasked = decltype(masked)::value;
        const bool valid = !kMasked || iv < nvec;
        static_assert(kFineShift == 16, "tkey is a multiple of 2^16");
        if constexpr (LG) {
            // Raw logits first (NaN never passes); weights only for those
            // at or above xb.
            float mx = VecT<VEC>::get(x, 0);
#pragma unroll
            for (int e = 1; e < VEC; ++e) mx = fmaxf(mx, VecT<VEC>::get(x, e));
            if (__builtin_amdgcn_ballot_w64(valid & (mx >= xb)) == 0) return;
        } else {
            if (__builtin_amdgcn_ballot_w64(valid & any_at_least<VEC>(x, (int)tkey)) == 0) return;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            u32 b = __float_as_uint(VecT<VEC>::get(x, e));
            if constexpr (LG) {
                const float xv = VecT<VEC>::get(x, e);
                b = xv >= xb ? __float_as_uint(logit_weight(xf, xv)) : 0u;
            }
            // Passing bits are keys: no sanitising.
            const u64 m = __builtin_amdgcn_ballot_w64(valid & (b - tkey <= span));
            if (m) {
                // Past the region's last slot, entries land on that slot and
                // the count reports the overflow.
                if (valid & (b - tkey <= span))
                    reg[min(wfill + mbcnt64(m), kRegion - 1)] = composite(b, (v0 + iv) * VEC + e);
                wfill += (u32)__popcll(m);
            }
        }
    };
    // Steps [0, nfull) have every lane inside the part; a partial last step
    // (its vector loaded up front) is appended after the loop.  Every step
    // issues exactly one refill load (clamped into the part), so the compiler
    // can count the loads in flight and wait for one at a time; steps from
    // nfull on append nothing in the loop.
    const u32 nfull = nvec / kBlock;
    for (u32 r0 = 0; r0 < nfull; r0 += kStreamDepth) {
#pragma unroll
        for (u32 d = 0; d < kStreamDepth; ++d) {
            if (r0 + d < nfull) append(std::false_type{}, pf[d], (r0 + d) * kBlock + threadIdx.x);
            pf[d] = ld_stream(&rv[min((r0 + d + kStreamDepth) * kBlock + threadIdx.x, last)]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (nfull * kBlock < nvec) append(std::true_type{}, tailv, nfull * kBlock + threadIdx.x);
    // Pack the regions: wave w's entries move to the offset of the waves below.
    if (lane_id() == 0) s.gn[wave] = wfill;
    __syncthreads();
    u32 fill = 0, before = 0;
    bool over = false;
#pragma unroll
    for (u32 w = 0; w < (u32)kWaves; ++w) {
        const u32 cw = uni(s.gn[w]);
        over |= cw > kRegion - 1;
        fill += cw;
        before += w < wave ? cw : 0u;
    }
    // A whole row headed for the binned finish leaves its entries in the
    // regions (that finish reads them there); otherwise the regions are
    // packed together.
    const bool direct =
        S == 1 && !over && fill >= k && !no_tkey && !(p.flags & TES_FLAG_TINY_BUFFER);
    if (!direct) {
        constexpr int kPerLane = kRegion / 64;
        u64 mine[kPerLane];
        const u32 nmine = wfill < kRegion ? wfill : kRegion;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const u32 i = lane_id() + 64u * j;
            mine[j] = i < nmine ? reg[i] : 0ull;
        }
        __syncthreads();
        if (!over) {
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const u32 i = lane_id() + 64u * j;
                if (i < nmine) sbuf(s)[before + i] = mine[j];
            }
        }
        __syncthreads();
    }
    tq = stat_phase(p, r, 13, tq);
    stat_phase(p, r, 8, tp);
    const u64 P = fixed_p(top_p);
    const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
    u32 tbase = tkey;
    if (S > 1) {
        // Publish this part, then the last part to arrive joins every part's
        // candidates at or above the largest threshold T.
        RowState* rs = ws_state(p, r);
        HalfPub* mine = half_pub(p, r, h);
        over = over || fill > kHalfCap;
        if (!over) {
            u64* dst = half_cands(p, r, h);
            for (u32 i = threadIdx.x; i < fill; i += kBlock) st_dev(&dst[i], sbuf(s)[i]);
        }
        if (threadIdx.x == 0) {
            st_dev(&mine->fill, fill);
            st_dev(&mine->tkey, tkey);
            st_dev(&mine->over, over ? 1u : 0u);
        }
        if (!arrive_last(s, &rs->ticket, S)) return;
        if (threadIdx.x < S) {
            const HalfPub* hp = half_pub(p, r, threadIdx.x);
            s.gn[threadIdx.x] = ld_g(&hp->fill);
            s.gn[kMaxSplit + threadIdx.x] = ld_g(&hp->tkey);
            s.gn[2 * kMaxSplit + threadIdx.x] = ld_g(&hp->over);
        }
        if (threadIdx.x == 0) {
            st_dev(&rs->ticket, 0u);
            s.ctr[3] = 0;
        }
        __syncthreads();
        u32 tmax = 0;
        over = false;
        for (u32 q = 0; q < S; ++q) {
            tmax = max(tmax, uni(s.gn[kMaxSplit + q]));
            over = over || uni(s.gn[2 * kMaxSplit + q]) != 0;
        }
        // Every entry of the row at or above T is in some part's candidates.
        // The parts' lists are read as one index space, eight loads per
        // thread in flight per round (one round for up to 4096 candidates).
        if (!over) {
            u32 pre[kMaxSplit + 1];
            pre[0] = 0;
            for (u32 q = 0; q < kMaxSplit; ++q) pre[q + 1] = pre[q] + (q < S ? uni(s.gn[q]) : 0u);
            const u32 total = pre[kMaxSplit];
            constexpr int kL = 8;
            for (u32 t0 = 0; t0 < total; t0 += kL * kBlock) {
                u64 c[kL];
                bool in[kL];
#pragma unroll
                for (int j = 0; j < kL; ++j) {
                    const u32 t = t0 + (u32)j * kBlock + threadIdx.x;
                    u32 q = 0;
#pragma unroll
                    for (u32 b = 1; b < kMaxSplit; ++b) q += t >= pre[b] ? 1u : 0u;
                    in[j] = t < total;
                    c[j] = in[j] ? ld_g(&half_cands(p, r, q)[t - pre[q]]) : 0ull;
                }
#pragma unroll
                for (int j = 0; j < kL; ++j)
                    wave_append(sbuf(s), in[j] && comp_key(c[j]) >= tmax, c[j], &s.ctr[3], 0,
                                kSlabCap);
            }
        }
        __syncthreads();
        fill = uni(s.ctr[3]);
        __syncthreads();
        over = over || fill > kSlabCap;
        tbase = tmax;
    }
    // Every part streamed every positive key (thresholds of sampled parts
    // are bin edges, far above 1) and nothing overflowed: the buffer holds
    // all of the row's positive entries.
    const bool all_pos = !over && tbase == 1u;
    if (!over && fill >= k) {
        // (At least k entries at or above the threshold: the row's best k are
        // among them.  Every positive key: no bin base for the binned finish.)
        slab_finish<LG>(s, r, fill, k, tbase > 1u ? tbase : 0u, P, u, direct ? wfill : ~0u);
    } else if (all_pos) {
        slab_short<VEC, LG>(s, r, fill, k, P, u, kPathSlab);
    } else {
        // A whole row that counted at least k entries at or above its
        // threshold has its best k there; anything else starts from 1.
        slab_restream<VEC, LG>(s, r, k, (S == 1 && !no_tkey && fill >= k) ? tkey : 1u, P, u);
    }
}

// The buffer sbuf(s)[0, n), k <= n <= kSlabCap, holds the row's best k (and
// every entry with key >= tkey).  The binned finish decides most rows; the
// others (and every row under TES_FLAG_TINY_BUFFER) cut the buffer to exactly
// the best k when it holds more than a sort takes, sort it descending (padded
// with zeros, which sort last) and finish on the first k positions.
template <bool MINP>
__device__ __forceinline__ void slab_finish(Smem& s, u32 r, u32 n, u32 k, u32 tkey, u64 P, u64 u,
                                         u32 wfill, u32 path, u64 c_k) {
    const Params p = params_from(s);
    const u64 tp = p.stats ? wall_clock64() : 0;
    const u32 gathered = n;
    const float theta = (MINP && p.min_p) ? ld_g(&p.min_p[r]) : 0.0f;
    // wfill != ~0u: the entries are still in the stream's wave regions (this
    // wave's count), and the binned finish packs them.
    if (!(p.flags & TES_FLAG_TINY_BUFFER) && tkey > 0) {
        Outcome ob;
        if (binned_topk<MINP>(s, n, k, tkey, P, u, ob, wfill, theta)) {
            stat_phase(p, r, 9, tp);
            if (c_k != ~0ull) ob.c_k = c_k;
            u32 nl = kNoList;
            if ((p.flags & kFlagList) && ob.kind != kZeroRow) {
                // The binned finish left the n entries packed at the buffer's start.
                constexpr int J = kSlabCap / kBlock;
                u64 c[J];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const u32 i = threadIdx.x + (u32)j * kBlock;
                    c[j] = i < n ? sbuf(s)[i] : 0ull;
                }
                nl = emit_list<J>(s, p, r, c, (p.flags & kFlagSupport) ? ob.c_k : ob.c_keep);
            }
            finish_row(s, p, r, ob, path, gathered, nl);
            return;
        }
        stat_why(p, r, 64u);
    }
    if (n > kSelCap || ((p.flags & TES_FLAG_TINY_BUFFER) && n > k)) {
        n = keep_above(s, n, select_slab(s, n, k));
        stat_add(p, r, 3, 1);
    }
    const u32 pad = n <= kBlock ? kBlock : n <= 2 * kBlock ? 2 * kBlock : 4 * kBlock;
    for (u32 i = n + threadIdx.x; i < pad; i += kBlock) sbuf(s)[i] = 0;
    __syncthreads();
    u64 ts = stat_phase(p, r, 14, tp);
    Outcome o;
    u32 nl = kNoList;
    // The sorted entries (zeros past n) stay in the threads' registers.
    auto sorted = [&](auto& v) {
        constexpr int E = sizeof(v) / sizeof(u64);
        sort_desc<E>(s, v);
        ts = stat_phase(p, r, 15, ts);
        o = resolve_sorted<E, MINP>(s, v, k, P, u, theta);
        if ((p.flags & kFlagList) && o.kind != kZeroRow)
            nl = emit_list<E>(s, p, r, v,
                              (p.flags & kFlagSupport) ? (c_k != ~0ull ? c_k : o.c_k) : o.c_keep);
    };
    if (pad == kBlock) {
        u64 v[1];
        sorted(v);
    } else if (pad == 2 * kBlock) {
        u64 v[2];
        sorted(v);
    } else {
        u64 v[4];
        sorted(v);
    }
    stat_phase(p, r, 9, tp);
    if (c_k != ~0ull) o.c_k = c_k;
    finish_row(s, p, r, o, path, gathered, nl);
}

// ---------------------------------------------------------------------------
// Top-p-only rows (k >= V)
// ---------------------------------------------------------------------------
// Fine bins holding descending mass positions P[n], looked up among the
// exchanged fine bins of the listed coarse bins (bin -1 when the position's
// coarse bin is not listed); above[n] receives the mass of all higher fine
// bins.  One thread per listed fine bin.
template <int N>
__device__ __forceinline__ void fine_locate(Smem& s, int nlist, const u64 (&P)[N], int (&bin)[N],
                                            u64 (&above)[N]) {
    if (threadIdx.x < (u32)N) {
        s.loc_bin[threadIdx.x] = -1;
        s.loc_above[threadIdx.x] = 0;
    }
    __syncthreads();
    for (int i = (int)threadIdx.x; i < nlist * 16; i += kBlock) {
        const int j = i >> 4, f = i & 15;
        const int cb = s.flist[j];
        u64 a = s.cabove[cb];
        for (int g = 15; g > f; --g) a += s.finem[j * 16 + g];
        const u64 w = s.finem[i];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            if (a < P[n] && P[n] <= a + w) {
                s.loc_bin[n] = cb * 16 + f;
                s.loc_above[n] = a;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < N; ++n) {
        bin[n] = (int)uni((u32)s.loc_bin[n]);
        above[n] = uni(s.loc_above[n]);
    }
    __syncthreads();
}

// Inclusive prefix sums within each row of 16 lanes (all lanes active).
__device__ __forceinline__ u64 row16_incl_scan(u64 x) {
    x += dpp_shift64<0x111>(x);
    x += dpp_shift64<0x112>(x);
    x += dpp_shift64<0x114>(x);
    x += dpp_shift64<0x118>(x);
    return x;
}

// One wave, after the first exchange: writes s.cabove (descending exclusive
// prefix of the summed coarse masses) and finds the coarse bins holding the
// boundary position T and the draw positions t_lo + 1 and t_hi + 1, where t_hi
// uses the largest mass the boundary's coarse bin allows.  Results go to
// s.loc_bin: the boundary bin, the draw range's top and bottom bins.  Lane l
// owns bins 256 - 4l - i (i < 4), and lane 63 also bin 0.
__device__ __forceinline__ void coarse_plan_wave(Smem& s, u64 T, u64 u) {
    const u32 lane = lane_id();
    u64 m[5], cab[5];
    int bb[5];
    u64 loc = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        bb[i] = (i < 4 || lane == 63) ? kCoarseBins - 1 - 4 * (int)lane - i : -1;
        m[i] = bb[i] >= 0 ? s.coarse[bb[i]] : 0ull;
        loc += m[i];
    }
    u64 a = wave_incl_scan(loc) - loc;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        cab[i] = a;
        if (bb[i] >= 0) s.cabove[bb[i]] = a;
        a += m[i];
    }
    // Each lane reports its bin holding W (or -1); the wave takes the one lane.
    auto locate = [&](u64 W, u64& cab_out, u64& m_out) {
        int hit = -1;
        u64 hc = 0, hm = 0;
#pragma unroll
        for (int i = 0; i < 5; ++i)
            if (bb[i] >= 0 && cab[i] < W && W <= cab[i] + m[i]) {
                hit = bb[i];
                hc = cab[i];
                hm = m[i];
            }
        const u64 bm = __builtin_amdgcn_ballot_w64(hit >= 0);
        const u32 L = bm ? (u32)__builtin_ctzll(bm) : 0u;
        cab_out = read_lane(hc, L);
        m_out = read_lane(hm, L);
        return bm ? (int)__builtin_amdgcn_readlane(hit, (int)L) : 0;
    };
    u64 cT, mT, c1, m1;
    const int cbT = locate(T, cT, mT);
    const u64 t_lo = __umul64hi(u, T), t_hi = __umul64hi(u, cT + mT);
    const int chi = locate(t_lo + 1, c1, m1);
    const int clo = locate(t_hi + 1, c1, m1);
    if (lane == 0) {
        s.loc_bin[0] = cbT;
        s.loc_bin[1] = chi;
        s.loc_bin[2] = clo;
    }
}

// One wave, once the listed fine masses are summed: the fine bin holding T
// (in the first listed coarse bin) with the mass above it, then the fine bins
// holding the draw positions t_lo + 1 and t_hi + 1 (t_hi from the boundary
// fine bin's largest mass).  Each row of 16 lanes scans the fine masses of one
// listed coarse bin, highest fine bin first.  Results: s.loc_bin[0..2] = fbT,
// fine bin of t_lo + 1, of t_hi + 1 (-1 if not found), s.loc_above[0] = mass
// above fbT.
__device__ __forceinline__ void fine_plan_wave(Smem& s, int nlist, u64 T, u64 u) {
    const u32 lane = lane_id();
    const int f = 15 - (int)(lane & 15u);  // fine bin within the coarse bin
    const u32 row = lane >> 4;
    // Pass 1: row 0 scans the boundary's coarse bin (list entry 0).
    const int cb0 = s.flist[0];
    const u64 w0 = row == 0 ? s.finem[f] : 0ull;
    const u64 a0 = s.cabove[cb0] + row16_incl_scan(w0) - w0;
    const u64 bm0 = __builtin_amdgcn_ballot_w64(row == 0 && a0 < T && T <= a0 + w0);
    const u32 L0 = bm0 ? (u32)__builtin_ctzll(bm0) : 0u;
    const int fbT = bm0 ? cb0 * 16 + (15 - (int)L0) : -1;
    const u64 above_f = read_lane(a0, L0);
    const u64 U = above_f + read_lane(w0, L0);
    const u64 t_lo = __umul64hi(u, T), t_hi = __umul64hi(u, U);
    // The list entries whose coarse bins hold the two draw positions.
    const u64 W1 = t_lo + 1, W2 = t_hi + 1;
    const bool lj = (int)lane < nlist;
    const int cbl = lj ? s.flist[lane] : 0;
    const u64 cl = lj ? s.cabove[cbl] : 0ull, ml = lj ? s.coarse[cbl] : 0ull;
    const u64 b1 = __builtin_amdgcn_ballot_w64(lj && cl < W1 && W1 <= cl + ml);
    const u64 b2 = __builtin_amdgcn_ballot_w64(lj && cl < W2 && W2 <= cl + ml);
    const int j1 = b1 ? (int)__builtin_ctzll(b1) : -1, j2 = b2 ? (int)__builtin_ctzll(b2) : -1;
    // Pass 2: row 1 scans list entry j1 for W1, row 2 entry j2 for W2.
    const int jr = row == 1 ? j1 : (row == 2 ? j2 : -1);
    const u64 Wr = row == 1 ? W1 : W2;
    const u64 wr = jr >= 0 ? s.finem[jr * 16 + f] : 0ull;
    const u64 ar = (jr >= 0 ? s.cabove[s.flist[jr]] : 0ull) + row16_incl_scan(wr) - wr;
    const u64 bm = __builtin_amdgcn_ballot_w64(jr >= 0 && ar < Wr && Wr <= ar + wr);
    const u64 bm1 = bm & 0x00000000FFFF0000ull, bm2 = bm & 0x0000FFFF00000000ull;
    if (lane == 0) {
        s.loc_bin[0] = fbT;
        s.loc_above[0] = above_f;
        s.loc_bin[1] = bm1 ? s.flist[j1] * 16 + (15 - ((int)__builtin_ctzll(bm1) - 16)) : -1;
        s.loc_bin[2] = bm2 ? s.flist[j2] * 16 + (15 - ((int)__builtin_ctzll(bm2) - 32)) : -1;
    }
}

template <int VEC, bool LG>
__device__ __forceinline__ void full_finish(Smem& s, u32 r, u32 nseg, u32 kind, u64 nit, u64 T,
                                         u64 above_f, int fbT, int nlist, bool failed);

template <int VEC, bool LG>
__device__ __attribute__((always_inline)) void do_full(Smem& s, u32 r, u32 seg, u32 nseg) {
    const Params p = params_from(s);
    typedef typename VecT<VEC>::T VT;
    const RowXf xf = row_xf<LG>(p, r);
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row_ptr<VEC>(p.probs, r, p.V));
    const u32 sv = (p.nvec + nseg - 1) / nseg;
    const u32 v0 = seg * sv, v1 = min(v0 + sv, p.nvec);
    const bool tiny = p.flags & TES_FLAG_TINY_BUFFER;
    const u32 gcap = tiny ? 16u : kGSeg;
    const int dmax = tiny ? 1 : kDMax;
    RowState* rs = ws_state(p, r);
    const float top_p = ld_g(&p.top_p[r]);  // issued early: its latency hides behind the loads
    stat_start(p, r, nseg);
    u64 tp = p.stats ? wall_clock64() : 0;

    // The histogram is cleared first so that each vector is counted as soon
    // as its load returns (loads are issued, and waited for, in order).
    for (int i = (int)threadIdx.x - 1; i < kFineBins; i += kBlock) shfine(s)[i] = 0;
    __syncthreads();
    // Probability rows hold the segment in registers from here to the
    // candidate collection after the second publication.  Logit rows stream
    // it twice instead (their weights are computed where a vector is
    // consumed): the weights' arithmetic on top of the held segment would
    // exceed the registers, and the spills serialise the loads.
    VT x[LG ? 1 : kSlots<VEC>];
    if constexpr (!LG) {
#pragma unroll
        for (int d = 0; d < kSlots<VEC>; ++d) {
            const u32 i = v0 + d * kBlock + threadIdx.x;
            x[d] = ld_stream(&rv[i < v1 ? i : v1 - 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const float* seg_row = reinterpret_cast<const float*>(rv + v0);
    // Visits the segment: f(x, i, in) for each vector x (weights for logit
    // rows) of index i the thread holds (in: inside the segment).
    auto seg_each = [&](auto f) {
        if constexpr (LG) {
            for_each_vec<VEC, kPassDepth, true>(seg_row, v1 - v0, [&](const VT& w, u32 iv, bool valid) {
                f(w, v0 + iv, valid);
            }, xf);
        } else {
#pragma unroll
            for (int d = 0; d < kSlots<VEC>; ++d) {
                const u32 i = v0 + d * kBlock + threadIdx.x;
                f(x[d], i, i < v1);
            }
        }
    };
    // Branch-free binning of the raw bits (fine_hist_add).  The segment's
    // mass is the sum of the histogram, taken afterwards; +inf entries (and
    // NaN bits) show up as signed maxima >= +inf and are counted only by
    // waves that hold one.
    u64 ninf = 0;
    // Min-p on logit rows: the largest mass is that of the top weight 1
    // (2^32), so the floor and its key are known up front; the segment adds
    // up the mass of its entries at or above the floor's key as it bins them.
    u64 mf = 0;
    float theta = 0.0f;
    if constexpr (LG) theta = p.min_p ? ld_g(&p.min_p[r]) : 0.0f;
    const u32 kf = minp_key(minp_floor(theta, 1ull << 32));
    const bool minp = LG && kf > 1u;
    const int dslot = -1 - (int)lane_id();  // this lane's discard slot
    auto hist_vec = [&](const VT& w, bool in) {
        if (in) {
            int mx = kIntMin;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const u32 b = __float_as_uint(VecT<VEC>::get(w, e));
                mx = max(mx, (int)b);
                fine_hist_add(shfine(s), b, dslot);
                if (minp) mf += (b >= kf && b <= kInfKey) ? key_mass(b) : 0ull;
            }
            if (__ballot(mx >= (int)kInfKey)) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) ninf += __float_as_uint(VecT<VEC>::get(w, e)) == kInfKey;
            }
        }
    };
    seg_each([&](const VT& w, u32, bool in) { hist_vec(w, in); });
    // Accumulators of the exchanges (ordered by the barriers below).
    for (int i = threadIdx.x; i < kCoarseBins; i += kBlock) s.coarse[i] = 0;
    for (int i = threadIdx.x; i < kDMax * 16; i += kBlock) s.finem[i] = 0;
    if (threadIdx.x < 3) s.csum[threadIdx.x] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        u64& top = shfine(s)[kFineBins - 1];
        top = (top / kTopUnit) << 32;
    }
    __syncthreads();
    u64 M = 0;
    for (int i = threadIdx.x; i < kFineBins; i += kBlock) M += shfine(s)[i];
    M = block_sum(s, M);
    ninf = block_sum(s, ninf);
    if (minp) mf = block_sum(s, mf);
    tp = stat_phase(p, r, 8, tp);

    // First exchange: this segment's mass, +inf count and coarse histogram.
    PubC* pc = pub_c(p, r, seg);
    for (int b = threadIdx.x; b < kCoarseBins; b += kBlock) {
        u64 v = 0;
        const int f0 = b * 16, f1 = min(f0 + 16, kFineBins);
        for (int f = f0; f < f1; ++f) v += shfine(s)[f];
        st_dev(&pc->coarse[b], v);
    }
    if (threadIdx.x == 0) {
        st_dev(&pc->M, M);
        st_dev(&pc->ninf, ninf);
        st_dev(&pc->mf, mf);
    }
    // bf16 rows: the whole fine histogram goes out with the first exchange.
    // (A bf16 row's segments are per-entry bound and end late, so the second
    // exchange's wait costs them more than the stores; for fp32 rows the
    // stores cost the other rows' streams more than the wait: measured.)
    constexpr bool kFused = VEC == 8;
    if constexpr (kFused) {
        PubFF* pff = pub_ff(p, r, seg);
        for (int i = threadIdx.x; i < kFineBins; i += kBlock) st_dev(&pff->fine[i], shfine(s)[i]);
    }
    const bool ok = arrive_wait(s, &rs->arrive_a, nseg);
    tp = stat_phase(p, r, 9, tp);

    // Every segment sums the exchange and takes the same decisions.  The
    // counter was acquired, so the published words are read with ordinary
    // loads that can be in flight together.
    static_assert(sizeof(PubC) == 8 * (4 + kCoarseBins), "PubC is M, ninf, ng, mf, coarse[]");
    sum_words(reinterpret_cast<const u64*>(pub_c(p, r, 0)), sizeof(PubC) / 8, nseg, 4 + kCoarseBins,
              [&](u32 i, u64 v) {
                  if (i < 2) s.csum[i] = v;
                  else if (i == 3) s.csum[2] = v;
                  else if (i >= 4) s.coarse[i - 4] = v;
              });
    __syncthreads();
    const u64 Mt = uni(s.csum[0]);
    const u64 nit = uni(s.csum[1]);
    const u64 P = fixed_p(top_p);
    const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
    const u32 kind = nit > 0 ? kInfRow : (Mt == 0 ? kZeroRow : kNormal);
    u64 T = kind == kNormal ? topp_threshold(P, Mt) : 0;
    // Min-p: the kept set ends where the inclusive mass reaches min(T, the
    // mass at or above the floor), which every later step takes as its T.
    if (LG && kf > 1u) {
        const u64 Mf = uni(s.csum[2]);
        T = Mf < T ? Mf : T;
    }
    int nlist = 0;
    bool decidable = ok;
    if (ok && kind == kNormal) {
        if (wave_id() == 0) coarse_plan_wave(s, T, u);
        __syncthreads();
        const int cbT = (int)uni((u32)s.loc_bin[0]);
        const int chi = (int)uni((u32)s.loc_bin[1]), clo = (int)uni((u32)s.loc_bin[2]);
        // Listed coarse bins: the boundary bin, then the draw range's bins
        // that hold mass, highest first.  A bin without mass holds neither
        // position (a range from a few large entries down to the bulk of the
        // row is mostly empty bins).
        if (wave_id() == 0) {
            const u32 lane = lane_id();
            u32 q = 1;  // listed so far (wave-uniform)
            if (lane == 0) s.flist[0] = cbT;
            for (int b0 = chi; b0 >= clo; b0 -= 64) {
                const int b = b0 - (int)lane;  // lane 0 takes the highest bin
                const bool in = b >= clo && b != cbT && s.coarse[b] != 0;
                const u64 m = __builtin_amdgcn_ballot_w64(in);
                const u32 pos = q + mbcnt64(m);
                if (in && pos < (u32)dmax) s.flist[pos] = b;
                q += (u32)__popcll(m);
            }
            if (lane == 0) s.misc[6] = q;
        }
        __syncthreads();
        const int cnt = (int)uni(s.misc[6]);
        if (cnt > dmax) {
            decidable = false;
            stat_why(p, r, 2u | (u32)min(cnt, 255) << 8);
        } else {
            nlist = cnt;
            if constexpr (!kFused) {
                // Second exchange: this segment's fine bins of the listed coarse bins.
                PubF* pf = pub_f(p, r, seg);
                for (int i = threadIdx.x; i < nlist * 16; i += kBlock) {
                    const int fb = s.flist[i / 16] * 16 + (i % 16);
                    st_dev(&pf->fine[i / 16][i % 16], fb < kFineBins ? shfine(s)[fb] : (u64)0);
                }
            }
        }
    }
    if (!ok) stat_why(p, r, 1u);
    if (!decidable && threadIdx.x == 0)
        or_dev(&rs->flags, (u32)kFlagFail);
    tp = stat_phase(p, r, 10, tp);
    if constexpr (!kFused) arrive_only(s, &rs->arrive_b);
    // While the other segments' fine masses arrive, collect this segment's
    // entries of the listed coarse bins (a superset of the fine bins the
    // gather will want) into per-wave LDS regions; the fine publication above
    // was the region's last reader.
    constexpr u32 kSpecReg = kSlabCap / kWaves;  // entries per wave region
    const u32 wave = uni(wave_id());
    u32 sfill = 0;
    const bool spec = !kFused && nlist > 0 && !tiny;
    if (spec) {
        const int cb = s.flist[0];
        const int chi = s.flist[nlist > 1 ? 1 : 0], clo = s.flist[nlist - 1];
        auto ckey0 = [&](int c) { return (u32)(c * 16 + (int)kFineBase) << kFineShift; };
        auto ckey1 = [&](int c) {
            return c == kCoarseBins - 1 ? kInfKey + 1 : (u32)((c + 1) * 16 + (int)kFineBase) << kFineShift;
        };
        const u32 kB0 = ckey0(cb), wB = ckey1(cb) - kB0;
        const u32 kR0 = ckey0(min(clo, chi)), wR = ckey1(max(clo, chi)) - kR0;
        u64* sreg = sbuf(s) + wave * kSpecReg;
        auto collect = [&](const VT& w, u32 i, bool in) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const u32 b = __float_as_uint(VecT<VEC>::get(w, e));
                const bool take = in & ((b - kB0 < wB) | (b - kR0 < wR));
                const u64 m = __builtin_amdgcn_ballot_w64(take);
                if (m) {
                    if (in & ((b - kB0 < wB) | (b - kR0 < wR)))
                        sreg[min(sfill + mbcnt64(m), kSpecReg - 1)] = composite(b, i * VEC + e);
                    sfill += (u32)__popcll(m);
                }
            }
        };
        seg_each(collect);
        if (lane_id() == 0) s.gn[32 + wave] = sfill;  // read after the barriers below
    }
    bool failed = !ok || !decidable;
    if constexpr (!kFused) {
        const bool ok2 = wait_arrivals(s, &rs->arrive_b, nseg);
        if (!ok2) stat_why(p, r, 4u);
        if (threadIdx.x == 0) {
            if (!ok2)
                or_dev(&rs->flags, (u32)kFlagFail);
            s.misc[4] = (!ok2 || (ld_dev(&rs->flags) & kFlagFail)) ? 1u : 0u;
        }
        __syncthreads();
        failed = uni(s.misc[4]) != 0;
        __syncthreads();
    }
    tp = stat_phase(p, r, 11, tp);

    // Gather, from registers, the entries the last segment needs.
    int fbT = 0;
    u64 above_f = 0;
    u32 ng = 0;
    u64* garea = gather_area(p, r, seg);
    if (!failed && kind == kNormal) {
        static_assert(sizeof(PubF) == 8 * 16 * kDMax, "PubF is fine[kDMax][16]");
        if constexpr (kFused) {
            // The listed coarse bins' fine masses from the segments' whole
            // histograms (acquired with the first exchange).
            for (u32 i = threadIdx.x; i < (u32)nlist * 16; i += kBlock) {
                const int fb = s.flist[i / 16] * 16 + (int)(i % 16);
                u64 v = 0;
                if (fb < kFineBins) {
                    for (u32 q0 = 0; q0 < nseg; q0 += 4) {
                        u64 w[4];
#pragma unroll
                        for (u32 j = 0; j < 4; ++j)
                            w[j] = q0 + j < nseg ? ld_g(&pub_ff(p, r, q0 + j)->fine[fb]) : 0ull;
#pragma unroll
                        for (u32 j = 0; j < 4; ++j) v += w[j];
                    }
                }
                s.finem[i] = v;
            }
        } else {
            sum_words(reinterpret_cast<const u64*>(pub_f(p, r, 0)), sizeof(PubF) / 8, nseg,
                      (u32)nlist * 16, [&](u32 i, u64 v) { s.finem[i] = v; });
        }
        __syncthreads();
        if (wave_id() == 0) fine_plan_wave(s, nlist, T, u);
        __syncthreads();
        fbT = (int)uni((u32)s.loc_bin[0]);
        above_f = uni(s.loc_above[0]);
        const int fdhi = (int)uni((u32)s.loc_bin[1]), fdlo = (int)uni((u32)s.loc_bin[2]);
        if (fbT < 0 || fdhi < 0 || fdlo < 0) {
            // Cannot happen for consistent exchanges; decide by the slow path.
            stat_why(p, r, 8u);
            if (threadIdx.x == 0)
                or_dev(&rs->flags, (u32)kFlagFail);
        } else {
            // Fine bins are key ranges: the boundary bin and the draw range.
            // (The top fine bin ends at +inf inclusive: NaN and negative bits
            // lie above it and are never taken.)
            const u32 kT0 = (u32)(fbT + kFineBase) << kFineShift;
            const u32 kT1 = fbT == kFineBins - 1 ? kInfKey + 1 : (u32)(fbT + 1 + kFineBase) << kFineShift;
            const u32 kD0 = (u32)(fdlo + kFineBase) << kFineShift;
            const u32 kD1 = fdhi == kFineBins - 1 ? kInfKey + 1 : (u32)(fdhi + 1 + kFineBase) << kFineShift;
            const u32 wT = kT1 - kT0, wD = kD1 - kD0;
            auto pred = [&](u32 b) { return (b - kT0 < wT) | (b - kD0 < wD); };
            bool spec_ok = spec;
            if (spec) {
#pragma unroll
                for (u32 w = 0; w < (u32)kWaves; ++w) spec_ok &= uni(s.gn[32 + w]) <= kSpecReg - 1;
            }
            if (spec_ok)
                ng = filter_regions(s, kSpecReg, sfill, pred, garea, gcap);
            else
                ng = gather_seg<VEC>(s, seg_each, pred, garea, gcap);
        }
    } else if (!failed && kind == kInfRow) {
        ng = gather_seg<VEC>(s, seg_each, [&](u32 key) { return key == kInfKey; }, garea, gcap);
    }
    if (threadIdx.x == 0) st_dev(&pc->ng, (u64)ng);
    const bool last = arrive_last(s, &rs->ticket, nseg);
    stat_phase(p, r, 12, tp);
    if (last) full_finish<VEC, LG>(s, r, nseg, kind, nit, T, above_f, fbT, nlist, failed);
}

// Last segment of a top-p-only row: load every segment's gathered entries
// and finish.
template <int VEC, bool LG>
__device__ __forceinline__ void full_finish(Smem& s, u32 r, u32 nseg, u32 kind, u64 nit, u64 T,
                                         u64 above_f, int fbT, int nlist, bool failed) {
    const Params p = params_from(s);
    RowState* rs = ws_state(p, r);
    u64 tp = p.stats ? wall_clock64() : 0;
    const bool tiny = p.flags & TES_FLAG_TINY_BUFFER;
    const u32 gcap = tiny ? 16u : kGSeg;
    const u64 P = fixed_p(ld_g(&p.top_p[r]));
    const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
    // One round of loads: the gather counts, the row's flags and, for up to
    // eight segments, every gather area whatever its count turns out to be.
    static_assert(kGSeg == 512, "gather areas of 2^9 entries");
    const u32 gsh = tiny ? 4u : 9u;  // gcap = 2^gsh
    const u32 gmask = (1u << gsh) - 1;
    const u64* g0 = gather_area(p, r, 0);
    const u32 total = nseg << gsh;
    const u64 ngv = threadIdx.x < nseg ? ld_g(&pub_c(p, r, threadIdx.x)->ng) : 0;
    const u32 fl = threadIdx.x == 0 ? ld_dev(&rs->flags) : 0u;
    constexpr int kL = 8;
    u64 c[kL];
#pragma unroll
    for (int j = 0; j < kL; ++j) {
        const u32 t = j * kBlock + threadIdx.x;
        c[j] = t < total ? ld_g(&g0[(size_t)(t >> gsh) * kGSeg + (t & gmask)]) : 0;
    }
    if (threadIdx.x < nseg) s.gn[threadIdx.x] = (u32)(ngv < gcap ? ngv : gcap);
    if (threadIdx.x == 0) {
        s.misc[3] = fl;
        s.ctr[3] = 0;
    }
    // (Its barriers publish s.gn, s.misc[3] and s.ctr[3].)
    const u64 over = block_sum(s, (threadIdx.x < nseg && ngv > gcap) ? 1u : 0u);
    const bool fail = (uni(s.misc[3]) & kFlagFail) || over != 0 || failed;
    if (over) stat_why(p, r, 16u);
    // Appends the gathered entries (with composites in [lo, hi) when reloading
    // them from the gather areas) to the buffer and returns their number (more
    // than kSelCap: some were not written).  The first call takes the values
    // loaded above; they are dead afterwards, so nothing holds them across the
    // selects.
    auto collect = [&](bool reload, u64 lo, u64 hi) {
        if (threadIdx.x == 0) s.ctr[3] = 0;
        __syncthreads();
        if (!reload) {
#pragma unroll
            for (int j = 0; j < kL; ++j) {
                const u32 t = j * kBlock + threadIdx.x;
                const bool in = t < total && (t & gmask) < s.gn[t >> gsh];
                wave_append(sbuf(s), in, c[j], &s.ctr[3], 0, kSelCap);
            }
        }
        for (u32 t0 = reload ? 0u : kL * kBlock; t0 < total; t0 += kBlock) {
            const u32 t = t0 + threadIdx.x;
            const bool in = t < total && (t & gmask) < s.gn[t >> gsh];
            const u64 cc = in ? ld_g(&g0[(size_t)(t >> gsh) * kGSeg + (t & gmask)]) : 0;
            wave_append(sbuf(s), in && cc >= lo && cc < hi, cc, &s.ctr[3], 0, kSelCap);
        }
        __syncthreads();
        const u32 n = uni(s.ctr[3]);
        __syncthreads();
        return n;
    };
    u32 nall = 0;
    if (!fail && kind != kZeroRow) nall = collect(false, 0, kNoUpper);
    // More than a buffer's worth gathered (wide boundary and draw ranges):
    // the boundary and the draw are then selected from one fine bin's
    // entries at a time.
    const bool staged = !fail && kind == kNormal && nall > kSelCap;
    u64 tf = stat_phase(p, r, 14, tp);
    Outcome o{};
    u32 path = kPathFull;
    bool fb = fail || (nall > kSelCap && !staged);
    if (!fb && kind == kNormal) {
        u32 n1 = nall;
        if (staged) n1 = collect(true, fine_lo(fbT), fine_hi(fbT));
        fb = n1 > kSelCap;
        if (!fb) {
            const bool binned = !tiny && fbT < kFineBins - 1;
            const Sel sb = binned ? fine_select<VEC == 8>(s, n1, fbT, T - above_f)
                                  : select_buf(s, n1, T - above_f, true, fine_lo(fbT), fine_hi(fbT));
            tf = stat_phase(p, r, 15, tf);
            const u64 M_p = above_f + sb.above + key_mass(comp_key(sb.c));
            const u64 t = __umul64hi(u, M_p);
            int fdv[1];
            u64 adv[1];
            fine_locate(s, nlist, {t + 1}, fdv, adv);
            const int fd = fdv[0];
            const u64 above_d = adv[0];
            u32 n2 = n1;
            if (staged && fd != fbT) n2 = fd >= 0 ? collect(true, fine_lo(fd), fine_hi(fd)) : kSelCap + 1;
            fb = n2 > kSelCap;
            if (!fb) {
                const Sel sd = (!tiny && fd < kFineBins - 1)
                                   ? fine_select<VEC == 8>(s, n2, fd, t + 1 - above_d)
                                   : select_buf(s, n2, t + 1 - above_d, true, fine_lo(fd), fine_hi(fd));
                o.kind = kNormal;
                o.c_keep = sb.c;
                o.M_p = M_p;
                o.token = comp_index(sd.c);
            }
        }
    }
    if (!fail && fb) stat_why(p, r, 32u);
    if (fb) {
        o = resolve_row<VEC, LG>(s, row_ptr<VEC>(p.probs, r, p.V), p.nvec, p.V, p.V, P, u, kSelCap,
                                 row_xf<LG>(p, r), (LG && p.min_p) ? ld_g(&p.min_p[r]) : 0.0f);
        path = kPathFullFallback;
    } else if (kind == kNormal) {
        // decided above
    } else if (kind == kZeroRow) {
        o.kind = kZeroRow;
        o.token = 0;  // the support is the whole row: its smallest index
    } else if (kind == kInfRow) {
        const u64 m = nit;
        const u64 t = __umul64hi(u, m);
        o.kind = kInfRow;
        o.m = (u32)m;
        o.token = comp_index(select_buf(s, nall, t + 1, false).c);
        u64 mn = ~0ull;
        for (u32 i = threadIdx.x; i < nall; i += kBlock) mn = sbuf(s)[i] < mn ? sbuf(s)[i] : mn;
        o.c_keep = block_min(s, mn);
    }
    if (threadIdx.x == 0) {
        st_dev(&rs->arrive_a, 0u);
        st_dev(&rs->arrive_b, 0u);
        st_dev(&rs->ticket, 0u);
        st_dev(&rs->flags, 0u);
    }
    stat_phase(p, r, 13, tp);
    finish_row(s, p, r, o, path, nall);
}

// ---------------------------------------------------------------------------
// Top-p-only rows decided by one workgroup each
// ---------------------------------------------------------------------------
// When a launch holds more top-p-only segments than the device keeps resident
// workgroups (large batches of long rows, such as the speculative-verify
// shape), the segments of a row would wait for each other across rounds of
// dispatch.  Such rows are decided by one workgroup each, with no exchange,
// in one pass over the row:
//   * The pass visits the row's rounds (kBlock vectors each) interleaved, so
//     that any prefix of the visit is spread over the whole row, and builds
//     the exact fine mass histogram, the +inf count and the min-p mass.
//   * After 1/16, 1/4 and 1/2 of the row, the histogram so far predicts the
//     fine bins that can hold the boundary (where the descending cumulative
//     mass reaches T) and the draw (position u * M_p): the bins whose
//     cumulative mass so far lies within z = 4.5 standard errors of the
//     predicted fraction (binomial, with the effective size (sum x)^2 /
//     sum x^2 of the weights seen and the finite-population factor), the
//     draw's widened for the boundary's uncertainty and by a bin each side.
//     Each prediction is intersected with the previous one.  From the first
//     prediction on, every wave appends its entries of the predicted bins to
//     its own region of the row's exchange area (unused on this path; no
//     atomics), and a wave whose region is three quarters full drops what a
//     narrower prediction no longer holds.
//   * After the last prediction the rounds visited before the first one are
//     visited again, for their entries of the predicted bins only.
//   * T, the boundary's bin and the draw range then follow from the exact
//     histogram.  When the predictions covered the boundary's bin, the
//     boundary and the draw are selected among the appended entries (those
//     of the needed bins are moved into LDS in one read when they fit).  A
//     bin the predictions missed costs one more pass that appends exactly
//     the bins needed: the result is the same either way.
// An empty intersection or a full region restarts the predictions (the
// second visit then reaches further).  Entries beyond a region after the
// exact pass too go to the whole-row passes.
constexpr u32 kRowList = kCoarseBins;  // listed draw bins (s.coarse / s.cabove / s.finem)
// Rounds in flight in the row pass.
template <bool LG>
constexpr u32 kRowDepth = 8;
static_assert(kRowList <= kDMax * 16, "draw-bin masses fit s.finem");
static_assert(5 * kWaves <= kCoarseBins, "fused reductions fit s.coarse");

// The appended entries of a row: kWaves regions of `stride` slots at gbuf,
// wave w's first s.gn[w] slots in use (written by this workgroup before a
// barrier), taken as one sequence with eight loads per thread in flight.
// Calls g(c, vmask) for each thread's batch of eight (bit k of vmask: c[k]
// is an entry), the same number of times in every thread.
template <typename G>
__device__ __forceinline__ void for_each_gathered8(Smem& s, const u64* gbuf, u32 stride, G g) {
    u32 off[kWaves + 1];
    off[0] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) off[w + 1] = off[w] + uni(s.gn[w]);
    const u32 n = off[kWaves];
    for (u32 i0 = 0; i0 < n; i0 += 8 * kBlock) {
        u64 c[8];
        u32 vm = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const u32 i = i0 + k * kBlock + threadIdx.x;
            // slot of sequence entry i: region w holds entries [off[w], off[w + 1])
            u32 base = 0;
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                if (i >= off[w]) base = (u32)w * stride - off[w];
            c[k] = i < n ? ld_g(&gbuf[base + i]) : 0ull;
            vm |= i < n ? 1u << k : 0u;
        }
        g(c, vm);
    }
}
// The same, calling f(c, valid) for each entry.
template <typename F>
__device__ __forceinline__ void for_each_gathered(Smem& s, const u64* gbuf, u32 stride, F f) {
    for_each_gathered8(s, gbuf, stride, [&](const u64 (&c)[8], u32 vm) {
#pragma unroll
        for (int k = 0; k < 8; ++k) f(c[k], ((vm >> k) & 1u) != 0);
    });
}
// Appends the gathered entries that satisfy pred to sbuf(s) at s.ctr[3] (which
// the caller has cleared), up to kSelCap: one LDS atomic per wave and batch
// of eight (per-entry appends queued each batch behind eight round trips).
template <typename Pred>
__device__ __forceinline__ void append_gathered(Smem& s, const u64* gbuf, u32 stride, Pred pred) {
    for_each_gathered8(s, gbuf, stride, [&](const u64 (&c)[8], u32 vm) {
        u32 mask = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) mask |= (((vm >> k) & 1u) && pred(c[k])) ? 1u << k : 0u;
        wave_append_n<8>(sbuf(s), mask, c, &s.ctr[3], 0, kSelCap);
    });
}

// Select among the appended entries with composite in [lo, hi): at which the
// descending cumulative weight (mass, or one per entry) reaches W, with the
// weight above it.  Up to lcap of them are compacted into LDS and selected
// there (fine bin f >= 0 with mass weights takes the binned fine select).
// More of them sharing one key (a run of ties; every fine bin of a bf16 row
// is one value): the W-th weight lies in the entry of rank m = ceil(W / q)
// in index order, found through a 2048-bin count table over the top 11 of
// the ibits index bits.  More, in a fine bin with mass weights: a 2048-bin
// mass table over the next 11 key bits finds the sub-bin holding W.  Either
// way the entries of that one table bin are selected in LDS.  Otherwise a
// radix select reads the appended entries once per digit.
template <bool kTieFirst>
__device__ Sel gather_select(Smem& s, const u64* gbuf, u32 stride, u64 lo, u64 hi, int f, u64 W,
                             bool mass, u32 lcap, u32 ibits) {
    auto collect = [&](auto pred) -> u32 {
        if (threadIdx.x == 0) s.ctr[3] = 0;
        __syncthreads();
        append_gathered(s, gbuf, stride, [&](u64 c) { return c >= lo && c < hi && pred(c); });
        __syncthreads();
        const u32 n = uni(s.ctr[3]);
        __syncthreads();
        return n;
    };
    const u32 nb = collect([](u64) { return true; });
    if (nb <= lcap)
        return (f >= 0 && mass) ? fine_select<kTieFirst>(s, nb, f, W)
                                : select_buf(s, nb, W, mass, lo, hi);
    u64 kmn = ~0ull, kmx = 0;
    for_each_gathered(s, gbuf, stride, [&](u64 c, bool v) {
        const bool in = v && c >= lo && c < hi;
        kmn = in && comp_key(c) < kmn ? comp_key(c) : kmn;
        kmx = in && comp_key(c) > kmx ? comp_key(c) : kmx;
    });
    kmn = block_min(s, kmn);
    kmx = block_max(s, kmx);
    if (kmn == kmx) {
        // One key: equal weights q, and descending composites are ascending
        // indices, so the digit is taken from the complemented index.
        const u64 q = mass ? key_mass((u32)kmn) : 1ull;
        const u64 m = (W + q - 1) / q;
        const u32 sh = ibits > 11 ? ibits - 11 : 0u;
        u32* hc = shcnt(s);
        for (int b = threadIdx.x; b < 2048; b += kBlock) hc[b] = 0;
        __syncthreads();
        for_each_gathered(s, gbuf, stride, [&](u64 c, bool v) {
            hist_add(hc, nullptr, false, v && c >= lo && c < hi, ((u32)c >> sh) & 2047u, 0);
        });
        __syncthreads();
        auto cf = [&](int b) { return (u64)hc[b]; };
        const Digit g = find_desc(s, 2048, m, cf, cf);
        const u32 d = g.d;
        const u32 n2 = collect([&](u64 c) { return (((u32)c >> sh) & 2047u) == d; });
        if (n2 <= kSelCap) {
            const Sel r = select_buf(s, n2, m - g.above, false);
            return Sel{r.c, (m - 1) * q};
        }
    } else if (f >= 0 && mass) {
        constexpr int kSubShift = kFineShift - 11;
        u32* hc = shcnt(s);
        u64* hm = shmass(s);
        for (int b = threadIdx.x; b < 2048; b += kBlock) {
            hc[b] = 0;
            hm[b] = 0;
        }
        __syncthreads();
        for_each_gathered(s, gbuf, stride, [&](u64 c, bool v) {
            const u32 key = comp_key(c);
            hist_add(hc, hm, true, v && c >= lo && c < hi, (key >> kSubShift) & 2047u, key_mass(key));
        });
        __syncthreads();
        const Digit g = find_desc(s, 2048, W, [&](int b) { return hm[b]; },
                                  [&](int b) { return (u64)hc[b]; });
        const u32 d = g.d;
        const u32 n2 = collect([&](u64 c) { return ((comp_key(c) >> kSubShift) & 2047u) == d; });
        if (n2 <= kSelCap) {
            const Sel r = select_buf(s, n2, W - g.above, true);
            return Sel{r.c, g.above + r.above};
        }
    }
    // Sequence entry i of the appended entries (as for_each_gathered).
    u32 off[kWaves + 1];
    off[0] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) off[w + 1] = off[w] + uni(s.gn[w]);
    return radix_select(s, off[kWaves], [&](u32 i, u64& c) {
        u32 base = 0;
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            if (i >= off[w]) base = (u32)w * stride - off[w];
        c = ld_g(&gbuf[base + i]);
        return true;
    }, W, mass, lo, hi, shcnt(s), shmass(s));
}

// Key range [fkey0(f), fkey1(f)) of fine bin f (the top bin ends at +inf
// inclusive: NaN and negative bits lie above it and are never taken).
__device__ __forceinline__ u32 fkey0(int f) { return (u32)(f + (int)kFineBase) << kFineShift; }
__device__ __forceinline__ u32 fkey1(int f) {
    return f == kFineBins - 1 ? kInfKey + 1 : (u32)(f + 1 + (int)kFineBase) << kFineShift;
}

// Up to two key ranges [k, k + w) (w = 0: empty).
struct KeyWin {
    u32 k0, w0, k1, w1;
    __device__ bool has(u32 b) const { return (b - k0 < w0) | (b - k1 < w1); }
    // The wave's lanes whose b is inside (each compare's lane mask is its
    // ballot: no per-lane value is built).
    __device__ u64 ballot(u32 b) const {
        return __builtin_amdgcn_ballot_w64(b - k0 < w0) | __builtin_amdgcn_ballot_w64(b - k1 < w1);
    }
    __device__ bool covers(int f) const {
        const u32 a = fkey0(f), e = fkey1(f) - 1;
        return (a - k0 < w0 && e - k0 < w0) || (a - k1 < w1 && e - k1 < w1);
    }
};
__device__ __forceinline__ KeyWin bins_win(int a0, int b0, int a1, int b1) {
    KeyWin w{0, 0, 0, 0};
    if (a0 <= b0) w.k0 = fkey0(a0), w.w0 = fkey1(b0) - fkey0(a0);
    if (a1 <= b1) w.k1 = fkey0(a1), w.w1 = fkey1(b1) - fkey0(a1);
    return w;
}

// Streams visited rounds j in [0, jb) (jb a multiple of kRowDepth<LG>, read at
// every step: it may grow) of a row visited in interleaved order: eight lanes
// each walk one eighth of the row, so visited round j < nj is row round
// (j & 7) * S8 + (j >> 3) (S8 rounds per eighth; past the row: invalid) and
// visited round j >= nj is visited round j - nj again.  f(x, iv, valid,
// first) is called for every vector of each round by every thread (first:
// j < nj); tick(j) after every kRowDepth<LG> rounds (j rounds visited).
template <int VEC, bool LG, typename F, typename G>
__device__ __forceinline__ void stream_rounds(const float* __restrict__ row, u32 nvec, u32 S8,
                                              const u32& jb, F f, G tick, const RowXf& xf) {
    typedef typename VecT<VEC>::T VT;
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row);
    const u32 nr = (nvec + kBlock - 1) / kBlock;
    const u32 nj = 8 * S8;
    auto vec_of = [&](u32 j) -> u32 {
        const u32 jj = j < nj ? j : j - nj;
        const u32 rd = (jj & 7) * S8 + (jj >> 3);
        return (j < jb && rd < nr) ? rd * kBlock + threadIdx.x : nvec;
    };
    constexpr u32 kD = kRowDepth<LG>;
    VT pf[kD];
#pragma unroll
    for (u32 d = 0; d < kD; ++d) {
        pf[d] = ld_stream(&rv[min(vec_of(d), nvec - 1)]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (u32 j0 = 0; j0 < jb; j0 += kD) {
#pragma unroll
        for (u32 d = 0; d < kD; ++d) {
            const u32 iv = vec_of(j0 + d);
            f(xform<VEC, LG>(xf, pf[d]), iv, iv < nvec, j0 + d < nj);
            pf[d] = ld_stream(&rv[min(vec_of(j0 + d + kD), nvec - 1)]);
            __builtin_amdgcn_sched_barrier(0);
        }
        tick(j0 + kD);
    }
}

// A u64 as the nearest-ish float (two conversions and a fused add).
__device__ __forceinline__ float u64f(u64 x) {
    return fmaf((float)(u32)(x >> 32), 0x1p32f, (float)(u32)x);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int VEC, bool LG>
__device__ __attribute__((always_inline)) void do_rowtopp(Smem& s, u32 r) {
    const Params p = params_from(s);
    typedef typename VecT<VEC>::T VT;
    const RowXf xf = row_xf<LG>(p, r);
    const float* row = row_ptr<VEC>(p.probs, r, p.V);
    const float top_p = ld_g(&p.top_p[r]);
    float theta = 0.0f;
    if constexpr (LG) theta = p.min_p ? ld_g(&p.min_p[r]) : 0.0f;
    // Logit rows: the largest mass is that of the top weight 1 (2^32).
    const u32 kf = LG ? minp_key(minp_floor(theta, 1ull << 32)) : 0u;
    const bool minp = LG && kf > 1u;
    const bool tiny = p.flags & TES_FLAG_TINY_BUFFER;
    // Appended entries: one region of wcap slots per wave, filled without
    // atomics (each wave keeps its own count).
    // (Global address space throughout: a generic store would also count
    // against the LDS counter, so the histogram's LDS waits would wait for
    // the stores; measured 448 -> 209 us for bf16 rows of the
    // speculative-verify batch.)
    u64* gbuf = reinterpret_cast<u64*>(ws_row(p, r));
    const u32 wcap = (tiny ? 64u : (u32)(p.rowbytes / sizeof(u64))) / kWaves;
    TES_GLOBAL u64* wreg = gp(gbuf) + (size_t)wave_id() * wcap;
    u32 wcnt = 0;  // this wave's appended entries (may pass wcap: counted, not written)
    const u32 lcap = tiny ? 32u : kSelCap;
    const u32 ibits = 32u - (u32)__clz((int)max(p.V - 1u, 1u));  // bits of an index
    const u64 P = fixed_p(top_p);
    const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
    stat_start(p, r, 1);
    u64 tp = p.stats ? wall_clock64() : 0;
    if (threadIdx.x == 0) s.npass = 0;

    // Fine binning of the row, branch free (fine_hist_add, with this lane's
    // discard slot); the top bin is turned into count * 2^32 after the pass.
    const int dslot = -1 - (int)lane_id();
    auto bin_add = [&](u32 b) { fine_hist_add(shfine(s), b, dslot); };

    auto wb = [&](int b) { return shfine(s)[b]; };

    const u32 nr = (p.nvec + kBlock - 1) / kBlock;
    const u32 S8 = (nr + 7) / 8;
    const u32 nj = 8 * S8;  // visited rounds (some past the row when nr % 8 != 0)
    // Predictions after j1 = nj/16 (at least kRowDepth<LG>) rounds, then after
    // 4 j1 and 8 j1 (a quarter and half of the row).
    constexpr u32 kD = kRowDepth<LG>;
    const u32 j1 = max(kD, (nj / 16) / kD * kD);
    const bool predict = nr >= 32;
    u32 next_upd = predict ? j1 : ~0u;

    // Prediction state (uniform): the bin ranges [tl, th] (boundary) and
    // [dl, dh] (draw), or the +inf window; appended since round j_start.
    // Before any prediction the window is the top bin (keys from 1.0 up: a
    // probability row's entries of 1.0 or more, a logit row's entries at its
    // maximum), appended from the first round.  A row whose mass all lies
    // there (a logit row at temperature 0, a one-hot row) then needs no
    // prediction, even when no update sees its mass.
    constexpr int kTop = kFineBins - 1;
    int tl = kTop, th = kTop, dl = kTop, dh = kTop;
    KeyWin win = bins_win(tl, th, dl, dh);
    bool started = true, infwin = false;
    u32 j_start = 0;
    u64 ninf = 0, mf = 0;

    for (int i = (int)threadIdx.x - 1; i < kFineBins; i += kBlock) shfine(s)[i] = 0;
    __syncthreads();

    // Appends one entry position of a step: the lanes whose take is set (bm,
    // the wave's ballot of take) store their entry's composite at the wave's
    // count plus their rank among those lanes.  The ballots of a step's
    // window tests are its masks: nothing else is built per lane.
    auto append1 = [&](u64 bm, bool take, u32 b, u32 idx) {
        if (bm == 0) return;
        const u32 pos = wcnt + mbcnt64(bm);
        if (take && pos < wcap) wreg[pos] = composite(b, idx);
        wcnt += (u32)__popcll(bm);
    };
    // bf16 rows: appends this lane's entries c[e] with bit e of mask set, in
    // lane order from a prefix sum over the lanes' counts (for eight entries
    // a vector, per-entry ballots measured slower: 195 -> 201 us on the
    // speculative-verify batch).  One condition per store and a branch-free
    // position: nesting the position update under the condition measured 2x
    // slower.
    auto append_lanes = [&](u32 mask, const u64 (&c)[VEC]) {
        const u32 cnt = (u32)__popc(mask);
        u32 pre = 0, tot = 0;
#pragma unroll
        for (int b = 0; (1 << b) <= VEC; ++b) {
            const u64 bb = __ballot((cnt >> b) & 1u);
            pre += mbcnt64(bb) << b;
            tot += (u32)__popcll(bb) << b;
        }
        u32 pos = wcnt + pre;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const bool take = (mask >> e) & 1u;
            if (take && pos < wcap) wreg[pos] = c[e];
            pos += take ? 1u : 0u;
        }
        wcnt += tot;
    };
    // Appends the step's entries taken by in (inb: the wave's ballot of in).
    auto append_step = [&](const VT& x, u32 iv, bool valid, auto in, auto inb) {
        if constexpr (VEC == 8) {
            u32 mask = 0;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                mask |= (valid && in(__float_as_uint(VecT<VEC>::get(x, e)))) ? 1u << e : 0u;
            if (__ballot(mask != 0) == 0) return;
            u64 c[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                c[e] = composite(__float_as_uint(VecT<VEC>::get(x, e)), iv * VEC + e);
            append_lanes(mask, c);
        } else {
            const u64 vm = __builtin_amdgcn_ballot_w64(valid);
            bool tk[VEC];
            u64 bm[VEC];
            u64 any = 0;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const u32 b = __float_as_uint(VecT<VEC>::get(x, e));
                tk[e] = valid & in(b);
                bm[e] = inb(b) & vm;
                any |= bm[e];
            }
            if (any == 0) return;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                append1(bm[e], tk[e], __float_as_uint(VecT<VEC>::get(x, e)), iv * VEC + e);
        }
    };
    // Keeps, in place, this wave's appended entries inside win (one wave:
    // each chunk of 64 * 8 slots is loaded before any of its kept entries is
    // stored, and stores never pass the slots loaded).
    auto compact = [&]() {
        __threadfence_block();
        const u32 n = wcnt;
        u32 kept = 0;
        for (u32 c0 = 0; c0 < n; c0 += 8 * 64) {
            u64 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const u32 i = c0 + k * 64 + lane_id();
                v[k] = i < n ? wreg[i] : 0ull;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const u32 i = c0 + k * 64 + lane_id();
                const bool keep = i < n && win.has(comp_key(v[k]));
                const u64 bm = __ballot(keep);
                if (keep) wreg[kept + mbcnt64(bm)] = v[k];
                kept += (u32)__popcll(bm);
            }
        }
        wcnt = kept;
    };

    constexpr int kPer = (kFineBins + kBlock - 1) / kBlock;
    auto update = [&](u32 j) {
        // The whole workgroup waits on the prediction: its waves take issue
        // priority over the other workgroup's streaming waves meanwhile
        // (speculative-verify batch 208 -> 204 us).
        __builtin_amdgcn_s_setprio(2);
        __syncthreads();  // the histogram and the appends of rounds < j are complete
        // This thread's bins (descending, as find_desc takes them); the
        // waves' totals of the mass, +inf count, min-p mass and squares so
        // far and the thread's exclusive mass prefix take one barrier.
        // (The prediction is a heuristic: fp32 arithmetic is ample for it.)
        const int top = kFineBins - 1 - (int)threadIdx.x * kPer;
        u64 lm = 0;
        float x2 = 0.0f;  // sum of squared weights x = q / 2^32: a bin's mass times its middle weight
#pragma unroll
        for (int jj = 0; jj < kPer; ++jj) {
            if (top - jj >= 0) {
                const u64 m = shfine(s)[top - jj];
                lm += m;
                x2 += u64f(m) * 0x1p-32f * __uint_as_float(fkey0(top - jj) + (1u << (kFineShift - 1)));
            }
        }
        const u64 inc = wave_incl_scan(lm);
        const u64 w1 = wave_sum(ninf), w2 = minp ? wave_sum(mf) : 0ull;
        const float w3 = wave_sum_f32(x2);
        const u32 wv = wave_id();
        if (lane_id() == 63) s.coarse[5 * wv + 0] = inc;
        if (lane_id() == 0) {
            s.coarse[5 * wv + 1] = w1;
            s.coarse[5 * wv + 2] = w2;
            s.coarse[5 * wv + 3] = (u64)__float_as_uint(w3);
            s.coarse[5 * wv + 4] = wcnt > wcap;
        }
        __syncthreads();
        u64 Ms = 0, pre = 0, ni = 0, mfs = 0, over = 0;
        float sx2 = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const u64 tw = s.coarse[5 * w + 0];
            Ms += tw;
            pre += (u32)w < wv ? tw : 0ull;
            ni += s.coarse[5 * w + 1];
            mfs += s.coarse[5 * w + 2];
            sx2 += __uint_as_float((u32)s.coarse[5 * w + 3]);
            over += s.coarse[5 * w + 4];
        }
        Ms = uni(Ms), ni = uni(ni), mfs = uni(mfs);
        const u64 ex = pre + inc - lm;  // mass of the bins above this thread's
        const bool lost = uni(over) != 0;
        if (ni > 0) {
            // A +inf row keeps its +inf entries: append those from here on.
            if (!infwin || lost) {
                infwin = started = true;
                j_start = j;
                win = KeyWin{kInfKey, 1, 0, 0};
                wcnt = 0;
            }
        } else if (Ms > 0) {
            u64 Ts = topp_threshold(P, Ms);
            if (minp) Ts = mfs < Ts ? mfs : Ts;
            Ts = Ts < 1 ? 1 : Ts;
            const float Md = u64f(Ms);
            const float Mx = Md * 0x1p-32f;
            const float neff = sx2 > 0.0f ? fmaxf(1.0f, Mx * Mx / sx2) : 1.0f;
            // Share of the row not seen yet (entries per visited round).
            const float seen = fminf(1.0f, (float)j * (float)(kBlock * VEC) / (float)p.V);
            const float fpc = sqrtf(fmaxf(0.0f, 1.0f - seen));
            const float ud = u64f(u) * 0x1p-64f;
            const float FT = u64f(Ts) / Md, FD = ud * FT;
            const float sT = sqrtf(FT * (1.0f - FT) / neff) * fpc;
            const float sD = sqrtf(FD * (1.0f - FD) / neff) * fpc;
            // Standard errors of margin: narrower windows append fewer
            // entries, wider ones miss less (speculative-verify batch: z =
            // 4.5 199.4 us per call, 2 of 6,144 rows needing another pass
            // over 12 draws; 3.5 194.1 us, 5 rows; 3.0 190.7 us, 12 rows;
            // 2.5 188.6 us, 23 rows).
            constexpr float z = 3.0f;
            auto clampW = [&](float w) -> u64 {
                if (!(w >= 1.0f)) return 1ull;
                if (w >= Md) return Ms;
                const float hi = floorf(w * 0x1p-32f);
                return ((u64)(u32)hi << 32) + (u64)(u32)fmaxf(w - hi * 0x1p32f, 0.0f);
            };
            // Margins: the boundary's, and the draw's, which also moves with
            // the kept mass M_p (from T up to T plus the boundary bin's mass:
            // allowed for as twice the boundary margin, and one bin on either
            // side of the draw's range).
            const float mT = (z * sT + 2.0f / neff) * Md;
            const float Tf = u64f(Ts), td = ud * Tf;
            const float mD = (z * (sD + ud * sT) + 2.0f / neff) * Md + ud * 2.0f * mT;
            const u64 Wq[4] = {clampW(Tf - mT), clampW(Tf + mT), clampW(td - mD), clampW(td + mD)};
            // The bins where the cumulative mass reaches each target.
            u64 acc = ex;
#pragma unroll
            for (int jj = 0; jj < kPer; ++jj) {
                const int b = top - jj;
                if (b >= 0) {
                    const u64 w = shfine(s)[b];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (acc < Wq[k] && Wq[k] <= acc + w) s.loc_bin[k] = b;
                    acc += w;
                }
            }
            __syncthreads();
            const int nth = (int)uni((u32)s.loc_bin[0]), ntl = (int)uni((u32)s.loc_bin[1]);
            const int ndh = min((int)uni((u32)s.loc_bin[2]) + 1, kFineBins - 1);
            const int ndl = max((int)uni((u32)s.loc_bin[3]) - 1, 0);
            const int ttl = max(tl, ntl), tth = min(th, nth), tdl = max(dl, ndl), tdh = min(dh, ndh);
            if (!started || infwin || lost || (ttl > tth && tdl > tdh)) {
                // (Re)start: the appended entries are dropped.
                tl = ntl, th = nth, dl = ndl, dh = ndh;
                started = true;
                infwin = false;
                j_start = j;
                win = bins_win(tl, th, dl, dh);
                wcnt = 0;
            } else {
                const bool narrower = ttl != tl || tth != th || tdl != dl || tdh != dh;
                tl = ttl, th = tth, dl = tdl, dh = tdh;
                win = bins_win(tl, th, dl, dh);
                // A wave whose region is three quarters full drops what the
                // narrower prediction no longer needs.
                if (narrower && 4 * wcnt > 3 * wcap) compact();
            }
        }
        __syncthreads();
        __builtin_amdgcn_s_setprio(0);
        next_upd = next_upd == j1 ? 4 * j1 : (next_upd == 4 * j1 ? 8 * j1 : ~0u);
        if (next_upd != ~0u && next_upd >= nj) next_upd = ~0u;
    };

    // The pass: exact histogram, +inf count, min-p mass, predicted bins;
    // then, once the predictions are final, the rounds visited before the
    // first one again (their entries of the predicted bins only).
    u32 jend = nj;
    stream_rounds<VEC, LG>(row, p.nvec, S8, jend, [&](const VT& x, u32 iv, bool valid, bool first) {
        if (first) {
            // Branch free: a lane past the row adds nothing to the discard slot.
            int mx = kIntMin;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const u32 b = valid ? __float_as_uint(VecT<VEC>::get(x, e)) : 0u;
                mx = max(mx, (int)b);
                bin_add(b);
                if (minp) mf += (b >= kf && b <= kInfKey) ? key_mass(b) : 0ull;
            }
            if (mx >= (int)kInfKey) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) ninf += __float_as_uint(VecT<VEC>::get(x, e)) == kInfKey;
            }
        }
        // (The window tests follow the histogram: lane masks kept across its
        // branches would be copied through vector registers.)
        append_step(x, iv, valid, [&](u32 b) { return win.has(b); },
                    [&](u32 b) { return win.ballot(b); });
    }, [&](u32 j) {
        if (j == next_upd) {
            const u64 t0 = p.stats ? wall_clock64() : 0;
            update(j);
            jend = nj + (started ? j_start : 0);
            stat_phase(p, r, 9, t0);
        }
    }, xf);
    if (threadIdx.x == 0) ++s.npass;
    // Publishes the waves' counts to s.gn (and returns whether all fit).
    auto publish = [&]() -> bool {
        if (lane_id() == 0) s.gn[wave_id()] = wcnt;
        __syncthreads();
        u32 mx = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = max(mx, s.gn[w]);
        mx = uni(mx);
        __syncthreads();  // s.gn is rewritten by the next publication
        return mx <= wcap;
    };
    const bool fits = publish();
    if (threadIdx.x == 0) {
        u64& top = shfine(s)[kFineBins - 1];
        top = (top / kTopUnit) << 32;
    }
    __syncthreads();
    u64 M = 0;
    for (int i = threadIdx.x; i < kFineBins; i += kBlock) M += shfine(s)[i];
    M = block_sum(s, M);
    ninf = block_sum(s, ninf);
    if (minp) mf = block_sum(s, mf);
    const bool chain = started && fits;
    if (!chain) stat_why(p, r, 1u << 16);
    tp = stat_phase(p, r, 8, tp);

    // Appends the entries taken by pred to the waves' regions in one pass
    // over the row, from empty regions; returns whether every region held
    // its entries (the counts are in s.gn).
    auto take = [&](auto pred) {
        return [&, pred](const VT& x, u32 iv, bool valid) {
            append_step(x, iv, valid, pred,
                        [&](u32 b) { return __builtin_amdgcn_ballot_w64(pred(b)); });
        };
    };
    auto pass = [&](auto pred) -> bool {
        wcnt = 0;
        for_each_vec<VEC, kStreamDepth, LG>(row, p.nvec, take(pred), xf);
        if (threadIdx.x == 0) ++s.npass;
        return publish();
    };
    // (s.gn holds the last publication until the next one.)
    auto total = [&]() {
        u32 n = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) n += s.gn[w];
        return uni(n);
    };
    const u32 nfin = total();

    // Decide.
    Outcome o{};
    bool fb = false;
    u32 gathered = nfin;
    if (ninf > 0) {
        // +inf rows keep their +inf entries: the t-th in index order.
        const bool ok = (chain && infwin) || pass([](u32 b) { return b == kInfKey; });
        gathered = total();
        if (ok) {
            const u64 lo = (u64)kInfKey << 32, hi = (u64)(kInfKey + 1) << 32;
            const u64 t = __umul64hi(u, ninf);
            o.kind = kInfRow;
            o.m = (u32)ninf;
            o.token = comp_index(
                gather_select<VEC == 8>(s, gbuf, wcap, lo, hi, -1, t + 1, false, lcap, ibits).c);
            u64 mn = ~0ull;
            for_each_gathered(s, gbuf, wcap, [&](u64 c, bool v) {
                mn = (v && c >= lo && c < mn) ? c : mn;
            });
            o.c_keep = block_min(s, mn);
        } else {
            fb = true;
        }
    } else if (M == 0) {
        o.kind = kZeroRow;
        o.token = 0;  // the support is the whole row: its smallest index
    } else {
        u64 T = topp_threshold(P, M);
        // Min-p: the kept set ends where the inclusive mass reaches
        // min(T, the mass at or above the floor).
        if (minp) T = mf < T ? mf : T;
        // The boundary's bin (by T), then the bins of draw positions t_lo + 1
        // and t_hi + 1, which depend on it.
        int fbT, bhi, blo;  // the draw's fine bins: bhi >= blo >= fbT
        u64 aboveT, mT, t_lo, t_hi, above_hi;
        if constexpr (VEC == 8) {
            // (bf16 rows: three block-wide searches.  The one scan below made
            // their pass loop twice as slow through register allocation.)
            const Digit gT = find_desc(s, kFineBins, T, wb, wb);
            fbT = (int)gT.d;
            aboveT = gT.above;
            mT = uni(shfine(s)[fbT]);
            t_lo = __umul64hi(u, T), t_hi = __umul64hi(u, aboveT + mT);
            const Digit g1 = find_desc(s, kFineBins, t_lo + 1, wb, wb);
            const Digit g2 = find_desc(s, kFineBins, t_hi + 1, wb, wb);
            bhi = (int)g1.d, blo = (int)g2.d;
            above_hi = g1.above;
        } else {
            // One exclusive scan of this thread's bins (descending) serves the
            // three searches.
            const int top = kFineBins - 1 - (int)threadIdx.x * kPer;
            u64 local = 0;
#pragma unroll
            for (int jj = 0; jj < kPer; ++jj)
                if (top - jj >= 0) local += shfine(s)[top - jj];
            if (threadIdx.x == 0) {
                s.bc[0] = 0, s.bc[1] = 0;
                s.loc_bin[0] = 0, s.loc_bin[1] = 0;
                s.loc_above[0] = 0;
            }
            const u64 ex = block_excl_scan(s, local);  // (its barriers order the above)
            // The bin where the descending cumulative mass reaches W, and the
            // mass above it: put(b, above) by the one thread holding it.
            auto search = [&](u64 W, auto put) {
                u64 acc = ex;
#pragma unroll
                for (int jj = 0; jj < kPer; ++jj) {
                    const int b = top - jj;
                    if (b >= 0) {
                        const u64 w = shfine(s)[b];
                        if (acc < W && W <= acc + w) put(b, acc);
                        acc += w;
                    }
                }
            };
            search(T, [&](int b, u64 a) { s.bc[0] = (u64)b, s.bc[1] = a; });
            __syncthreads();
            fbT = (int)uni((u32)s.bc[0]);
            aboveT = uni(s.bc[1]);
            mT = uni(shfine(s)[fbT]);
            t_lo = __umul64hi(u, T), t_hi = __umul64hi(u, aboveT + mT);
            search(t_lo + 1, [&](int b, u64 a) { s.loc_bin[0] = b, s.loc_above[0] = a; });
            search(t_hi + 1, [&](int b, u64) { s.loc_bin[1] = b; });
            __syncthreads();
            bhi = (int)uni((u32)s.loc_bin[0]), blo = (int)uni((u32)s.loc_bin[1]);
            above_hi = uni(s.loc_above[0]);
            __syncthreads();
        }
        // The non-empty bins of [blo, bhi] with their masses and the mass
        // above each, highest first (one wave, 64 bins per step).
        if (wave_id() == 0) {
            const u32 lane = lane_id();
            u64 base = above_hi;
            u32 q = 0;
            for (int b0 = bhi; b0 >= blo; b0 -= 64) {
                const int b = b0 - (int)lane;
                const bool in = b >= blo;
                const u64 m = in ? shfine(s)[b] : 0ull;
                const u64 inc = wave_incl_scan(m);
                const bool ne = in && m != 0;
                const u64 bm = __ballot(ne);
                const u32 pos = q + mbcnt64(bm);
                if (ne && pos < kRowList) {
                    s.coarse[pos] = (u64)b;
                    s.cabove[pos] = base + inc - m;
                    s.finem[pos] = m;
                }
                q += (u32)__popcll(bm);
                base += read_lane(inc, 63);
            }
            if (lane == 0) s.misc[6] = q;
        }
        __syncthreads();
        const u32 nlist = uni(s.misc[6]);
        tp = stat_phase(p, r, 10, tp);
        // Bins whose entries are all appended: inside both ha and hb.
        KeyWin need = bins_win(fbT, fbT, blo, bhi);
        // Bins whose entries are all appended: inside both ha and hb.
        KeyWin ha = need, hb = win;
        bool ok = chain && win.covers(fbT);
        if (!ok) {
            stat_why(p, r, 1u << 17);
            // One pass for the boundary's bin and the draw range; if they
            // overflow, the boundary's bin alone (the draw's follows).
            hb = KeyWin{0, 0xFFFFFFFFu, 0, 0};
            ok = nlist <= kRowList && pass([&](u32 b) { return need.has(b); });
            if (!ok) {
                need.w1 = 0;
                ok = pass([&](u32 b) { return need.has(b); });
            }
            ha = need;
        }
        gathered = total();
        fb = !ok;
        // One read of the appended entries puts those of the needed bins
        // into LDS when they fit; otherwise each select reads them.
        auto collect_need = [&]() -> u32 {
            if (threadIdx.x == 0) s.ctr[3] = 0;
            __syncthreads();
            append_gathered(s, gbuf, wcap,
                            [&](u64 c) { return ha.has(comp_key(c)) && hb.has(comp_key(c)); });
            __syncthreads();
            const u32 n = uni(s.ctr[3]);
            __syncthreads();
            return n;
        };
        auto select_bin = [&](u32 nl, int f, u64 W) -> Sel {
            const bool bin = !tiny && f < kFineBins - 1;
            if (nl <= lcap)
                return bin ? fine_select<VEC == 8>(s, nl, f, W)
                           : select_buf(s, nl, W, true, fine_lo(f), fine_hi(f));
            return gather_select<VEC == 8>(s, gbuf, wcap, fine_lo(f), fine_hi(f), bin ? f : -1, W,
                                           true, lcap, ibits);
        };
        if (!fb) {
            u32 nl = collect_need();
            const Sel sb = select_bin(nl, fbT, T - aboveT);
            const u64 M_p = aboveT + sb.above + key_mass(comp_key(sb.c));
            const u64 t = __umul64hi(u, M_p);
            // The listed bin holding draw position t + 1.
            if (threadIdx.x == 0) {
                s.loc_bin[0] = -1;
                s.loc_above[0] = 0;
            }
            __syncthreads();
            for (u32 i = threadIdx.x; i < min(nlist, kRowList); i += kBlock) {
                const u64 a = s.cabove[i], m = s.finem[i];
                if (a < t + 1 && t + 1 <= a + m) {
                    s.loc_bin[0] = (int)s.coarse[i];
                    s.loc_above[0] = a;
                }
            }
            __syncthreads();
            const int fd = (int)uni((u32)s.loc_bin[0]);
            const u64 above_d = uni(s.loc_above[0]);
            __syncthreads();
            if (fd < 0) {
                fb = true;  // the draw lies outside the listed bins: not for a consistent histogram
            } else {
                if (!(ha.covers(fd) && hb.covers(fd))) {
                    stat_why(p, r, 1u << 18);
                    ha = bins_win(fd, fd, 0, -1);
                    hb = KeyWin{0, 0xFFFFFFFFu, 0, 0};
                    ok = pass([&](u32 b) { return ha.has(b); });
                    gathered = total();
                    if (ok) nl = collect_need();
                }
                fb = !ok;
                if (!fb) {
                    const Sel sd = select_bin(nl, fd, t + 1 - above_d);
                    o.kind = kNormal;
                    o.c_keep = sb.c;
                    o.M_p = M_p;
                    o.token = comp_index(sd.c);
                }
            }
        }
    }
    u32 path = kPathFullRow;
    if (fb) {
        stat_why(p, r, 1u << 19);
        o = resolve_row<VEC, LG>(s, row, p.nvec, p.V, p.V, P, u, kSelCap, xf, theta);
        path = kPathFullFallback;
    }
    stat_add(p, r, 3, uni(s.npass));
    stat_phase(p, r, 13, tp);
    finish_row(s, p, r, o, path, gathered);
}

// ---------------------------------------------------------------------------
// Whole-row items
// ---------------------------------------------------------------------------
template <int VEC, bool LG>
__device__ __attribute__((always_inline)) void do_whole(Smem& s, u32 r, u32 k_eff) {
    const Params p = params_from(s);
    stat_start(p, r, 1);
    const u64 P = fixed_p(ld_g(&p.top_p[r]));
    const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
    const bool tiny = p.flags & TES_FLAG_TINY_BUFFER;
    if (threadIdx.x == 0) s.npass = 0;
    const Outcome o = resolve_row<VEC, LG>(s, row_ptr<VEC>(p.probs, r, p.V), p.nvec, p.V, k_eff, P,
                                           u, tiny ? 64u : kSelCap, row_xf<LG>(p, r),
                                           (LG && p.min_p) ? ld_g(&p.min_p[r]) : 0.0f);
    stat_add(p, r, 3, uni(s.npass));
    finish_row(s, p, r, o, kPathWhole, 0);
}

// ---------------------------------------------------------------------------
// Main kernel
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32 row_k_eff(const Params& p, u32 r) {
    const int32_t k = ld_g(&p.top_k[r]);
    return (k <= 0 || (u32)k >= p.V) ? p.V : (u32)k;
}

__device__ __forceinline__ u32 row_class(const Params& p, u32 k_eff, u32 s_full) {
    if (p.flags & TES_FLAG_FORCE_ROW_SELECT) return kClsWhole;
    if (k_eff == 1) return kClsGreedy;
    if (k_eff <= kSlabMaxK) return kClsSlab;
    if (k_eff == p.V && s_full <= p.s_ws) return kClsFull;
    return kClsWhole;
}

// One work item per workgroup, in block order.  Items [0, nf * S) are the
// segments of the nf top-p-only rows, S consecutive items per row: blocks are
// dispatched in order, so the segments of a row start together and wait for
// each other only briefly (the waits are bounded all the same).  When the
// launch's items would not all be resident at once, S is 1 and each such
// row is decided by its one workgroup (one pass, no exchange).  The other
// rows follow, one item each: whole-row rows, top-k rows, then greedy rows.
// Blocks beyond the last item return at once.  No item loop: values live
// across one would raise the register pressure of every path.
template <int VEC, bool LG>
__global__ __launch_bounds__(kBlock, kWavesPerSimd) void tes_main_kernel(Params p) {
    __shared__ Smem s;
    if (threadIdx.x == 0) {
        s.p = p;
        s.npass = 0;
    }
    const u32 s_full = (p.nvec + p.seg_vec_full - 1) / p.seg_vec_full;

    // Rows in class order (stable within a class): each thread takes two rows.
    const u32 r0 = threadIdx.x * 2;
    u32 cls[2];
    u64 local = 0;  // four 16-bit class counts
    for (int j = 0; j < 2; ++j) {
        const u32 r = r0 + j;
        const u32 ke = r < p.rows ? row_k_eff(p, r) : 0u;
        cls[j] = r < p.rows ? row_class(p, ke, s_full) : 4u;
        if (cls[j] == kClsSlab) s.slab_k[r] = (u16)ke;
        if (cls[j] < 4) local += 1ull << (16 * cls[j]);
    }
    const u64 ex = block_excl_scan(s, local);
    if (threadIdx.x == kBlock - 1) {
        const u64 tot = ex + local;
        s.misc[0] = (u32)(tot & 0xFFFF);
        s.misc[1] = (u32)((tot >> 16) & 0xFFFF);
        s.misc[2] = (u32)((tot >> 32) & 0xFFFF);
        s.misc[3] = (u32)((tot >> 48) & 0xFFFF);
    }
    __syncthreads();
    u32 base[4];
    u32 acc = 0;
    for (int c = 0; c < 4; ++c) {
        base[c] = acc;
        acc += s.misc[c];
    }
    u32 seen[4] = {0, 0, 0, 0};
    for (int j = 0; j < 2; ++j) {
        const u32 c = cls[j];
        if (c < 4) {
            s.rows[base[c] + (u32)((ex >> (16 * c)) & 0xFFFF) + seen[c]] = (u16)(r0 + j);
            ++seen[c];
        }
    }
    __syncthreads();
    const u32 nf = uni(s.misc[kClsFull]);
    const u32 n_whole = uni(s.misc[kClsWhole]);
    const u32 n_slab = uni(s.misc[kClsSlab]);
    const u32 n_greedy = uni(s.misc[kClsGreedy]);
    // Top-k rows are split into S parts only when every item, parts included,
    // is resident at once (parts that wait for a slot only delay their rows);
    // greedy rows too when there is still room.  Parts after the first come
    // last in block order.
    // Top-p-only rows are cut into s_full segments while every item of the
    // launch is resident at once; otherwise each is decided by one
    // workgroup in one pass over the row (or under TES_FLAG_ROW_TOPP).
    const bool row_topp = (p.flags & TES_FLAG_ROW_TOPP) ||
                          nf * s_full + n_whole + n_slab + n_greedy > p.slots;
    const u32 segs = row_topp ? 1u : s_full;
    const u32 base_items = nf * segs + n_whole + n_slab + n_greedy;
    // Parts beyond half the resident slots cost more in joins than they gain
    // (measured), so the split stops there.
    const u32 room = p.slots / 2;
    u32 S = 1, Sg = 1;
    for (u32 c = p.split; c > 1 && S == 1; --c)
        if (base_items + (c - 1) * n_slab <= room) S = c;
    for (u32 c = S; c > 1 && Sg == 1; --c)
        if (base_items + (S - 1) * n_slab + (c - 1) * n_greedy <= room) Sg = c;
    const u32 full_end = nf * segs;
    const u32 whole_end = full_end + n_whole;
    const u32 first_end = whole_end + n_slab;
    const u32 greedy_end = first_end + n_greedy * Sg;
    const u32 item = blockIdx.x;
    __syncthreads();
    if (item < full_end) {
        if (row_topp) {
            do_rowtopp<VEC, LG>(s, uni((u32)s.rows[item]));
        } else {
            const u32 j = item / s_full;
            do_full<VEC, LG>(s, uni((u32)s.rows[j]), item - j * s_full, s_full);
        }
    } else if (item < whole_end) {
        const u32 r = uni((u32)s.rows[nf + (item - full_end)]);
        do_whole<VEC, LG>(s, r, row_k_eff(p, r));
    } else if (item < first_end) {
        const u32 r = uni((u32)s.rows[nf + n_whole + (item - whole_end)]);
        do_slab<VEC, LG>(s, r, s.slab_k[r], 0, S);
    } else if (item < greedy_end) {
        const u32 i = (item - first_end) / Sg;
        const u32 r = uni((u32)s.rows[nf + n_whole + n_slab + i]);
        // Greedy rows yield bandwidth when the launch fills at least half
        // the resident slots (below that HBM is not saturated and yielding
        // only slows them: B=128 with 64 greedy rows 24.4 -> 27.2 us) and
        // they make up at most three quarters of the rows (measured: 75%
        // greedy B=256 batch 41.3 -> 36.9 us, hetero batch 40.7 -> 39.4 us;
        // an all-greedy batch keeps 29 us).
        do_greedy<VEC, LG>(s, r, item - first_end - i * Sg, Sg,
                       n_greedy <= 3 * (n_slab + nf + n_whole) && 2 * base_items >= p.slots);
    } else if (item < greedy_end + n_slab * (S - 1)) {
        const u32 i = (item - greedy_end) % n_slab, h = 1 + (item - greedy_end) / n_slab;
        const u32 r = uni((u32)s.rows[nf + n_whole + i]);
        do_slab<VEC, LG>(s, r, s.slab_k[r], h, S);
    }
}

// renorm_out[r][i] = q_i / M_p for kept entries (1/m for kept +inf), else 0
// (q from the weights for logit rows).  Each workgroup writes one contiguous
// range of at most kRenormSpan entries of a row.  A row with a list is
// written without being read: the list's kept entries (>= c_keep) in the
// range are stored by the threads that read them from the list and marked in
// an LDS bitmap, then the range's other entries are stored as zeros (each
// entry has one writer).  Rows without a list are read, and each entry
// tested against c_keep.
constexpr u32 kRenormSpan = 32768;
template <int VEC, bool LG>
__global__ __launch_bounds__(256) void tes_renorm_kernel(Params p, const Decision* __restrict__ dec,
                                                         float* __restrict__ out) {
    typedef typename VecT<VEC>::T VT;
    __shared__ u32 marks[kRenormSpan / 32];
    const u32 r = blockIdx.y;
    const u32 V = p.V, nvec = p.nvec;
    const Decision d = dec[r];
    const u32 per = (nvec + gridDim.x - 1) / gridDim.x;
    const u32 v0 = min(blockIdx.x * per, nvec), v1 = min(v0 + per, nvec);
    float* __restrict__ orow = out + (size_t)r * V;
    const double inv = d.kind == kNormal ? 1.0 / (double)d.M_p : 0.0;
    const float w_inf = d.kind == kInfRow ? (float)(1.0 / (double)d.m) : 0.0f;
    auto value = [&](u32 key) {
        return d.kind == kInfRow ? w_inf : (float)((double)key_mass(key) * inv);
    };
    auto store = [&](u32 iv, const float (&o)[VEC]) {
        if constexpr (VEC == 4) {
            reinterpret_cast<f4*>(orow)[iv] = f4{o[0], o[1], o[2], o[3]};
        } else if constexpr (VEC == 8) {
            reinterpret_cast<f4*>(orow)[2 * iv] = f4{o[0], o[1], o[2], o[3]};
            reinterpret_cast<f4*>(orow)[2 * iv + 1] = f4{o[4], o[5], o[6], o[7]};
        } else {
            orow[iv] = o[0];
        }
    };
    if (d.nlist != kNoList && (v1 - v0) * VEC <= kRenormSpan) {
        const u32 e0 = v0 * VEC, e1 = v1 * VEC;
        for (u32 i = threadIdx.x; i < kRenormSpan / 32; i += 256) marks[i] = 0;
        __syncthreads();
        const u64* list = row_list(p, r);
        for (u32 i = threadIdx.x; i < d.nlist; i += 256) {
            const u64 c = ld_g(&list[i]);
            const u32 idx = comp_index(c);
            if (c >= d.c_keep && idx >= e0 && idx < e1) {
                atomicOr(&marks[(idx - e0) >> 5], 1u << ((idx - e0) & 31));
                orow[idx] = value(comp_key(c));
            }
        }
        __syncthreads();
        for (u32 iv = v0 + threadIdx.x; iv < v1; iv += 256) {
            const u32 off = (iv - v0) * VEC;
            const u32 m = (marks[off >> 5] >> (off & 31)) & ((1u << VEC) - 1u);
            if (m == 0) {
                const float z[VEC] = {};
                store(iv, z);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (!((m >> e) & 1u)) orow[(size_t)iv * VEC + e] = 0.0f;
            }
        }
        return;
    }
    const RowXf xf = row_xf<LG>(p, r);
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row_ptr<VEC>(p.probs, r, V));
    for (u32 iv = v0 + threadIdx.x; iv < v1; iv += 256) {
        const VT x = xform<VEC, LG>(xf, rv[iv]);
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const u32 key = sanitize(__float_as_uint(VecT<VEC>::get(x, e)));
            const bool kept = d.kind != kZeroRow && composite(key, iv * VEC + e) >= d.c_keep;
            o[e] = kept ? value(key) : 0.0f;
        }
        store(iv, o);
    }
}



// ---------------------------------------------------------------------------
// Speculative verification epilogue
// ---------------------------------------------------------------------------
// SonicSampler paper, appendix C.4, eqs. (15)-(16), with its draft-to-target
// mapping.  The target rows of a launch have already been decided by the
// sampling kernel (their Decisions hold each row's final distribution): p(x)
// = q_x / M_p on the kept entries of a normal row, 1 / m on the kept +inf
// entries of a +inf row, 1 on the token of a zero-mass row.  S workgroups
// per request (S = 1 when requests fill the device):
//   * wave 0 of each tests the L drafts at once, lane l: the draft's mass
//     Q = floor(min(y_d, 1) * 2^32) in its draft row, p(d) = num / den in
//     target row pi(l), and u * Q * den <= num * 2^96 with u = words 2 and 3
//     of that row's Philox block, compared on three 64-bit limbs;
//   * the first rejected position l draws its correction from
//     R_x = max(0, num_x * 2^32 - Q_x * den) (the residual of eq. (16) scaled
//     by 2^32 den): t = floor(u R / 2^64) with u = words 0 and 1 (the row's
//     own draw, whose token is not used then), and the correction is the
//     first x in vocabulary order whose inclusive prefix of R exceeds t.
//     With S > 1 each wave sums R over its eighth of its workgroup's S-th
//     of the vocabulary and publishes it; the last workgroup to arrive
//     keeps the part holding t.  Within the range, a workgroup splits it in
//     eight, one eighth per wave (each wave sums its eighth's R; the eighth
//     holding t is kept), until the range is one vector per thread, then a
//     workgroup scan.  R = 0 (p <= q everywhere) takes the row's own token;
//   * with every draft accepted, the bonus token is target row pi(L)'s own
//     token.
// A request whose map or draft tokens are out of range gets accept_len -1
// and tokens -1.
struct SpecArgs {
    const float* draft;      // [nreq][L][V] draft probabilities (fp32)
    const int32_t* tokens;   // [nreq][L] draft tokens
    const int32_t* map;      // [nreq][L + 1] target row of each position, or null
    int32_t* out;            // [nreq][L + 1] output tokens
    int32_t* accept;         // [nreq] accepted drafts
    u32 L;
    u32 Lt;                  // target rows per request
};

__device__ __forceinline__ Decision load_decision(const Params& p, u32 r) {
    const Decision* d = ws_decision(p, r);
    Decision o;
    o.kind = ld_g(&d->kind);
    o.m = ld_g(&d->m);
    o.token = ld_g(&d->token);
    o.path = ld_g(&d->path);
    o.c_keep = ld_g(&d->c_keep);
    o.M_p = ld_g(&d->M_p);
    o.c_k = ld_g(&d->c_k);
    return o;
}

// Row r's p(x) = num / den from its Decision and entry x's key.
__device__ __forceinline__ u64 dist_num(const Decision& d, u32 key, u32 x) {
    if (d.kind == kZeroRow) return x == d.token ? 1ull : 0ull;
    if (composite(key, x) < d.c_keep) return 0;
    return d.kind == kInfRow ? 1ull : key_mass(key);
}
__device__ __forceinline__ u64 dist_den(const Decision& d) {
    return d.kind == kNormal ? d.M_p : (d.kind == kInfRow ? (u64)d.m : 1ull);
}

// u * Q * den <= num * 2^96 on 64-bit limbs (Q <= 2^32, den < 2^51, num <= 2^32).
__device__ __forceinline__ bool draft_accepted(u64 u, u64 Q, u64 den, u64 num) {
    const u64 m0 = u * Q, m1 = __umul64hi(u, Q);  // u Q = m1:m0, m1 < 2^32
    const u64 p0 = m0 * den, c0 = __umul64hi(m0, den);
    const u64 t1 = m1 * den, t2 = __umul64hi(m1, den);
    const u64 p1 = t1 + c0;
    const u64 p2 = t2 + (p1 < t1 ? 1ull : 0ull);  // u Q den = p2:p1:p0
    const u64 r2 = num >> 32, r1 = num << 32;     // num 2^96 = r2:r1:0
    if (p2 != r2) return p2 < r2;
    if (p1 != r1) return p1 < r1;
    return p0 == 0;
}

typedef unsigned __int128 u128;

// R_x as hi / lo 32-bit parts of a value <= 2^64: hi = R >> 32 (<= 2^32),
// lo = R & (2^32 - 1); sums of up to 2^18 of each stay below 2^51.
__device__ __forceinline__ void residual_parts(u64 num, u64 Q, u64 den, u64& hi, u64& lo) {
    const u64 a1 = num >> 32, a0 = num << 32;              // num 2^32
    const u64 b0 = Q * den, b1 = __umul64hi(Q, den);       // Q den
    const bool pos = a1 > b1 || (a1 == b1 && a0 > b0);
    const u64 d0 = a0 - b0, d1 = a1 - b1 - (a0 < b0 ? 1ull : 0ull);  // a - b when pos
    hi = pos ? ((d1 << 32) | (d0 >> 32)) : 0ull;
    lo = pos ? (d0 & 0xFFFFFFFFull) : 0ull;
}
__device__ __forceinline__ u128 from_parts(u64 hi, u64 lo) { return ((u128)hi << 32) + lo; }

template <int VEC>
__global__ __launch_bounds__(kBlock) void tes_verify_kernel(Params p, SpecArgs a) {
    typedef typename VecT<VEC>::T VT;
    __shared__ u64 wsum[2][kWaves];
    __shared__ u64 wpart[kWaves];
    __shared__ u32 res[4];
    const u32 n = blockIdx.x;
    const u32 lane = lane_id(), wave = wave_id();
    const u32 L = a.L, Lt = a.Lt, V = p.V;
    int32_t* out = a.out + (size_t)n * (L + 1);
    // Wave 0: validate the request, test every draft, find the first rejection.
    if (wave == 0) {
        const u32 l = lane;
        int j = 0;
        bool bad = false;
        if (l <= L) {
            j = a.map ? ld_g(&a.map[(size_t)n * (L + 1) + l]) : (int)l;
            bad = j < 0 || (u32)j >= Lt;
        }
        int32_t d = 0;
        if (l < L) {
            d = ld_g(&a.tokens[(size_t)n * L + l]);
            bad = bad || d < 0 || (u32)d >= V;
        }
        const bool any_bad = __ballot(bad) != 0;
        bool acc = true;
        if (!any_bad && l < L) {
            const u32 r = n * Lt + (u32)j;
            const Decision dec = load_decision(p, r);
            const float* trow = row_ptr<1>(p.probs, r, V);
            const u32 key = sanitize(__float_as_uint(ld_g(&trow[d])));
            const float* drow = a.draft + ((size_t)n * L + l) * V;
            const u64 Q = key_mass(sanitize(__float_as_uint(ld_g(&drow[d]))));
            const u64 ua = philox_uniform<true>(p.seed, p.row_base + r, p.offset);
            acc = draft_accepted(ua, Q, dist_den(dec), dist_num(dec, key, (u32)d));
        }
        const u64 rej = __ballot(l < L && !acc);
        const u32 first = rej ? (u32)__builtin_ctzll(rej) : L;  // accepted drafts
        const u32 jf = (u32)__builtin_amdgcn_readlane(j, (int)(first < 64 ? first : 0));
        // (Every chunk's workgroup takes the same decisions; chunk 0 writes them.)
        const bool writer = blockIdx.y == 0;
        if (any_bad) {
            if (writer && l <= L) out[l] = -1;
            if (writer && l == 0) a.accept[n] = -1;
        } else {
            if (writer && l < first) out[l] = d;
            if (writer && l > first && l <= L) out[l] = -1;
            if (l == 0) {
                if (writer) a.accept[n] = (int32_t)first;
                res[0] = first;
                res[1] = n * Lt + jf;  // the row of the rejection, or of the bonus
                if (writer && first == L)
                    out[L] = (int32_t)ld_g(&ws_decision(p, n * Lt + jf)->token);
            }
        }
        if (l == 0) res[2] = any_bad ? 1u : 0u;
    }
    __syncthreads();
    const u32 first = res[0];
    if (res[2] != 0 || first >= L) return;  // marked, or every draft accepted (bonus written)
    // The correction at position `first`, from target row r and draft row `first`.
    const u32 r = res[1];
    const Decision dec = load_decision(p, r);
    const u64 den = dist_den(dec);
    const VT* __restrict__ tv = reinterpret_cast<const VT*>(row_ptr<VEC>(p.probs, r, V));
    const VT* __restrict__ dv =
        reinterpret_cast<const VT*>(a.draft + ((size_t)n * L + first) * V);
    // Residual parts of vector iv, summed over its entries.
    auto vec_parts = [&](u32 iv, u64& hi, u64& lo) {
        const VT x = ld_g(&tv[iv]);
        const VT y = ld_g(&dv[iv]);
        hi = lo = 0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const u32 key = sanitize(__float_as_uint(VecT<VEC>::get(x, e)));
            const u64 Q = key_mass(sanitize(__float_as_uint(VecT<VEC>::get(y, e))));
            u64 h, l2;
            residual_parts(dist_num(dec, key, iv * VEC + e), Q, den, h, l2);
            hi += h;
            lo += l2;
        }
    };
    u32 v0 = 0, v1 = p.nvec;
    u128 t = 0;
    bool have_t = false;
    const u32 S = gridDim.y;
    if (S > 1) {
        // The vocabulary is cut into S chunks, one workgroup each, and each
        // chunk into eighths, one wave each: every wave sums its eighth's
        // residual and publishes it in the exchange area of the request's
        // first target row; the last workgroup to arrive locates t among the
        // 8 S parts and searches on within its part.
        const u32 cv = (p.nvec + S - 1) / S;
        const u32 c0 = min(blockIdx.y * cv, p.nvec), c1 = min(c0 + cv, p.nvec);
        const u32 sub = (cv + kWaves - 1) / kWaves;
        const u32 w0 = min(c0 + wave * sub, c1), w1 = min(w0 + sub, c1);
        u64 hi = 0, lo = 0;
#pragma unroll 4
        for (u32 iv = w0 + lane; iv < w1; iv += 64) {
            u64 h, l2;
            vec_parts(iv, h, l2);
            hi += h;
            lo += l2;
        }
        hi = wave_sum(hi);
        lo = wave_sum(lo);
        u64* pub = reinterpret_cast<u64*>(ws_row(p, n * Lt));
        const u32 part = blockIdx.y * kWaves + wave;
        if (lane == 0) {
            st_dev(&pub[2 * part], hi);
            st_dev(&pub[2 * part + 1], lo);
        }
        vm_wait();
        __syncthreads();
        RowState* rs = ws_state(p, n * Lt);
        if (threadIdx.x == 0) {
            const u32 tk = add_dev(&rs->vticket, 1u);
            res[3] = tk == S - 1 ? 1u : 0u;
            if (tk == S - 1) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                st_dev(&rs->vticket, 0u);  // zero between calls
            }
        }
        __syncthreads();
        if (res[3] == 0) return;
        // Parts in order: wave 0 holds parts lane, 64 + lane (S * 8 <= 64).
        static_assert(kWaves * 8 <= 64, "every part fits one wave's lanes");
        const u32 np = S * kWaves;
        if (wave == 0) {
            const u64 ph = lane < np ? ld_g(&pub[2 * lane]) : 0ull;
            const u64 pl = lane < np ? ld_g(&pub[2 * lane + 1]) : 0ull;
            // Inclusive prefix of the parts as u128 from the 32-bit-part sums.
            const u64 ih = wave_incl_scan(ph), il = wave_incl_scan(pl);
            const u128 inc = from_parts(ih, il), own = from_parts(ph, pl);
            const u128 all = from_parts(read_lane(ih, 63), read_lane(il, 63));
            u128 tt = 0;
            if (all != 0) {
                const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
                tt = (u128)u * (u64)(all >> 64) + __umul64hi(u, (u64)all);
            }
            // The part whose inclusive prefix first exceeds t.
            const u64 hit = __ballot(lane < np && all != 0 && inc > tt);
            const u32 k = hit ? (u32)__builtin_ctzll(hit) : 0u;
            const u128 before = inc - own;
            if (lane == k) {
                res[0] = all == 0 ? 1u : 0u;
                wsum[0][0] = (u64)(tt - before);
                wsum[0][1] = (u64)((tt - before) >> 64);
                res[1] = k;
            }
        }
        __syncthreads();
        if (res[0] != 0) {  // p <= q everywhere: the row's own token
            if (threadIdx.x == 0) out[first] = (int32_t)dec.token;
            return;
        }
        t = ((u128)wsum[0][1] << 64) | wsum[0][0];
        have_t = true;
        // Part k: eighth k % 8 of chunk k / 8, as its wave summed it.
        const u32 k = res[1];
        const u32 q0 = min((k / kWaves) * cv, p.nvec), q1 = min(q0 + cv, p.nvec);
        v0 = min(q0 + (k % kWaves) * sub, q1);
        v1 = min(v0 + sub, q1);
        __syncthreads();
    }
    while (true) {
        const u32 nv = v1 - v0;
        if (nv <= kBlock) break;
        // Each wave sums one eighth of the range.
        const u32 sub = (nv + kWaves - 1) / kWaves;
        const u32 w0 = min(v0 + wave * sub, v1), w1 = min(w0 + sub, v1);
        u64 hi = 0, lo = 0;
#pragma unroll 4
        for (u32 iv = w0 + lane; iv < w1; iv += 64) {
            u64 h, l2;
            vec_parts(iv, h, l2);
            hi += h;
            lo += l2;
        }
        hi = wave_sum(hi);
        lo = wave_sum(lo);
        if (lane == 0) {
            wsum[0][wave] = hi;
            wsum[1][wave] = lo;
        }
        __syncthreads();
        u128 tot[kWaves];
        u128 all = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            tot[w] = from_parts(wsum[0][w], wsum[1][w]);
            all += tot[w];
        }
        __syncthreads();
        if (!have_t) {
            if (all == 0) {  // p <= q everywhere: the row's own token
                if (threadIdx.x == 0) out[first] = (int32_t)dec.token;
                return;
            }
            // t = floor(u * R / 2^64), R = all < 2^83.
            const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
            const u64 R0 = (u64)all, R1 = (u64)(all >> 64);
            const u64 c = __umul64hi(u, R0);
            t = (u128)u * R1 + c;
            have_t = true;
        }
        u32 k = 0;
        u128 before = 0;
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w) {
            if (k == (u32)w && before + tot[w] <= t) {
                before += tot[w];
                k = (u32)w + 1;
            }
        }
        t -= before;
        const u32 n0 = min(v0 + k * sub, v1);
        v1 = min(n0 + sub, v1);
        v0 = n0;
    }
    // One vector per thread: a workgroup scan of the residual parts.
    const u32 iv = v0 + threadIdx.x;
    u64 hi = 0, lo = 0;
    if (iv < v1) vec_parts(iv, hi, lo);
    if (!have_t) {
        // The whole row fits one round: its total decides t.
        const u64 th = block_sum_u64(wpart, hi), tl = block_sum_u64(wpart, lo);
        const u128 all = from_parts(th, tl);
        if (all == 0) {
            if (threadIdx.x == 0) out[first] = (int32_t)dec.token;
            return;
        }
        const u64 u = philox_uniform(p.seed, p.row_base + r, p.offset);
        t = (u128)u * (u64)(all >> 64) + __umul64hi(u, (u64)all);
    }
    const u64 eh = block_excl_scan_u64(wpart, hi), el = block_excl_scan_u64(wpart, lo);
    const u128 pre = from_parts(eh, el), own = from_parts(hi, lo);
    if (threadIdx.x == 0) res[3] = 0xFFFFFFFFu;
    __syncthreads();
    if (iv < v1 && pre <= t && t < pre + own) {
        const VT x = ld_g(&tv[iv]);
        const VT y = ld_g(&dv[iv]);
        u128 acc = pre;
        u32 hit = iv * VEC + VEC - 1;
        for (int e = 0; e < VEC; ++e) {
            const u32 key = sanitize(__float_as_uint(VecT<VEC>::get(x, e)));
            const u64 Q = key_mass(sanitize(__float_as_uint(VecT<VEC>::get(y, e))));
            u64 h, l2;
            residual_parts(dist_num(dec, key, iv * VEC + e), Q, den, h, l2);
            acc += from_parts(h, l2);
            if (acc > t) {
                hit = iv * VEC + e;
                break;
            }
        }
        res[3] = hit;
    }
    __syncthreads();
    if (threadIdx.x == 0) out[first] = (int32_t)res[3];
}

// Logit rows: the maximum of each of p.xparts parts of every row (NaN counts
// as -inf), as an order-preserving u32 encoding (sign bit set for
// non-negative values, all bits inverted for negative ones), so that the
// sampling kernel takes the row maximum as the largest of the parts.
template <int VEC>
__global__ __launch_bounds__(256) void tes_rowmax_kernel(Params p) {
    typedef typename VecT<VEC>::T VT;
    static_assert(VEC == 4 || VEC == 1, "logit rows are fp32");
    const u32 r = blockIdx.y, part = blockIdx.x;
    const u32 pv = (p.nvec + p.xparts - 1) / p.xparts;
    const u32 v0 = part * pv, v1 = min(v0 + pv, p.nvec);
    const VT* __restrict__ rv = reinterpret_cast<const VT*>(row_ptr<VEC>(p.probs, r, p.V));
    auto enc = [](float x) {
        const u32 b = x != x ? 0xFF800000u : __float_as_uint(x);
        return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    };
    u32 e = 0;
    constexpr u32 kU = 4;
    for (u32 i0 = v0; i0 < v1; i0 += kU * 256) {
        VT x[kU];
#pragma unroll
        for (u32 j = 0; j < kU; ++j) {
            const u32 iv = i0 + j * 256 + threadIdx.x;
            x[j] = ld_stream(&rv[iv < v1 ? iv : v1 - 1]);
        }
#pragma unroll
        for (u32 j = 0; j < kU; ++j) {
            u32 m = enc(VecT<VEC>::get(x[j], 0));
            for (int c = 1; c < VEC; ++c) m = max(m, enc(VecT<VEC>::get(x[j], c)));
            e = max(e, m);
        }
    }
    __shared__ u32 wm[4];
    u32 m = e;
#pragma unroll
    for (u32 o = 32; o >= 1; o >>= 1) m = max(m, lane_xor(m, o));
    if (lane_id() == 0) wm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        *gp(&ws_xmax(p, r)->part[part]) = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
}

// Slab export: one workgroup per row writes the row's support in its sorted
// order (descending probability, ascending index, the order in which the
// cake_sampling page emits its slab) with the renormalised weight of each
// entry (the renorm_out value at that index), for supports of at most `cap`
// entries; other rows get length -1.  The support is every entry whose
// composite is at least the row's boundary c_k (the whole row when k_eff = V):
// a row whose support list holds it all loads the list, others collect it in
// one pass over the row; it is then sorted by a bitonic network in LDS.
constexpr int kSlabThreads = 512;
constexpr u32 kSlabExportMax = 1024;

template <int VEC>
__global__ __launch_bounds__(kSlabThreads) void tes_slab_kernel(
    const float* __restrict__ probs, u32 V, u32 nvec, const int32_t* __restrict__ top_k,
    const Decision* __restrict__ dec, const unsigned char* __restrict__ lists, u32 list_stride,
    u32 cap, int32_t* __restrict__ slab_index, float* __restrict__ slab_renorm,
    int32_t* __restrict__ slab_len, u32* __restrict__ route) {
    typedef typename VecT<VEC>::T VT;
    static_assert(kSlabThreads == kBlock && kSlabExportMax == 2 * kBlock, "the register sort's shape");
    __shared__ u64 buf[2 * kSlabExportMax];  // the support, then the sort's two halves
    __shared__ u32 cnt;
    const u32 r = blockIdx.x;
    const Decision d = dec[r];
    const int32_t kr = top_k[r];
    const u32 k_eff = (kr <= 0 || (u32)kr >= V) ? V : (u32)kr;
    int32_t* oi = slab_index + (size_t)r * cap;
    float* ow = slab_renorm + (size_t)r * cap;
    if (threadIdx.x == 0) {
        if (route) route[r] = d.path;
        slab_len[r] = k_eff <= cap ? (int32_t)k_eff : -1;
        cnt = 0;
    }
    if (k_eff > cap) {
        for (u32 j = threadIdx.x; j < cap; j += kSlabThreads) {
            oi[j] = -1;
            ow[j] = 0.0f;
        }
        return;
    }
    const u64 lo = k_eff == V ? 0ull : d.c_k;
    __syncthreads();
    if (k_eff == 1) {
        // A one-entry support is the boundary itself: no pass over the row.
        if (threadIdx.x == 0) {
            buf[0] = lo;
            cnt = 1;
        }
    } else if (d.nlist == k_eff) {
        // The row's support list holds its whole support: k_eff entries, all
        // >= c_k.  (A support list is shorter when zeros complete the
        // support, and empty for a row without mass.)
        const u64* __restrict__ list =
            reinterpret_cast<const u64*>(lists + (size_t)r * list_stride);
        for (u32 i = threadIdx.x; i < d.nlist; i += kSlabThreads) buf[i] = ld_g(&list[i]);
        if (threadIdx.x == 0) cnt = d.nlist;
    } else {
        // Eight loads per thread in flight: a single workgroup streams the row.
        const VT* __restrict__ rv = reinterpret_cast<const VT*>(row_ptr<VEC>(probs, r, V));
        constexpr u32 kU = 8;
        for (u32 i0 = 0; i0 < nvec; i0 += kU * kSlabThreads) {
            VT x[kU];
#pragma unroll
            for (u32 j = 0; j < kU; ++j) {
                const u32 iv = i0 + j * kSlabThreads + threadIdx.x;
                x[j] = ld_stream(&rv[iv < nvec ? iv : nvec - 1]);
            }
#pragma unroll
            for (u32 j = 0; j < kU; ++j) {
                const u32 iv = i0 + j * kSlabThreads + threadIdx.x;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const u64 c =
                        composite(sanitize(__float_as_uint(VecT<VEC>::get(x[j], e))), iv * VEC + e);
                    if (iv < nvec && c >= lo) {
                        const u32 pos = atomicAdd(&cnt, 1u);
                        if (pos < kSlabExportMax) buf[pos] = c;
                    }
                }
            }
        }
    }
    __syncthreads();
    const u32 n = cnt < k_eff ? cnt : k_eff;  // exactly k_eff for a consistent boundary
    // Descending sort of buf[0, n) padded with zeros (composites are unique;
    // zeros sort last), held in registers: kBlock or 2 kBlock positions.
    const u32 N = n <= kBlock ? kBlock : 2 * kBlock;
    for (u32 i = n + threadIdx.x; i < N; i += kSlabThreads) buf[i] = 0;
    __syncthreads();
    const double inv = d.kind == kNormal ? 1.0 / (double)d.M_p : 0.0;
    const float w_inf = d.kind == kInfRow ? (float)(1.0 / (double)d.m) : 0.0f;
    auto put = [&](u32 j, u64 c) {
        const u32 key = comp_key(c);
        const bool kept = d.kind != kZeroRow && c >= d.c_keep;
        oi[j] = (int32_t)comp_index(c);
        ow[j] = !kept ? 0.0f : (d.kind == kInfRow ? w_inf : (float)((double)key_mass(key) * inv));
    };
    auto write = [&](const auto& v) {
        constexpr u32 E = sizeof(v) / sizeof(u64);
#pragma unroll
        for (u32 e = 0; e < E; ++e) {
            const u32 j = threadIdx.x * E + e;
            if (j < n) put(j, v[e]);
        }
    };
    if (N == kBlock) {
        u64 v[1];
        sort_desc_buf<1>(buf, v);
        write(v);
    } else {
        u64 v[2];
        sort_desc_buf<2>(buf, v);
        write(v);
    }
    for (u32 j = n + threadIdx.x; j < cap; j += kSlabThreads) {
        oi[j] = -1;
        ow[j] = 0.0f;
    }
}

// Clears n words at p.  The statistics are cleared by this kernel rather
// than by a memset, so that a call that a caller captures into a HIP graph
// records kernel nodes only.
__global__ __launch_bounds__(256) void tes_clear_kernel(u32* __restrict__ p, u32 n) {
    for (u32 i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

// Reference stream: reads nvec 16-byte vectors once (coalesced, eight loads
// per thread in flight, non-temporal like the sampler's row loads) and folds
// them into one word, stored only when it equals a value no input is expected
// to produce, so that no load can be dropped.  Its duration over the same
// bytes is the plain read time the sampler's duration is compared with.
__global__ __launch_bounds__(256) void tes_read_kernel(const f4* __restrict__ src, u64 nvec,
                                                       u32* __restrict__ sink) {
    constexpr int kU = 8;
    const u64 stride = (u64)gridDim.x * 256u;
    u32 acc = 0;
    u64 i = (u64)blockIdx.x * 256u + threadIdx.x;
    for (; i + (kU - 1) * stride < nvec; i += kU * stride) {
        f4 v[kU];
#pragma unroll
        for (int j = 0; j < kU; ++j) v[j] = ld_stream(&src[i + j * stride]);
#pragma unroll
        for (int j = 0; j < kU; ++j)
            acc ^= __float_as_uint(v[j][0]) ^ __float_as_uint(v[j][1]) ^
                   __float_as_uint(v[j][2]) ^ __float_as_uint(v[j][3]);
    }
    for (; i < nvec; i += stride) {
        const f4 v = ld_stream(&src[i]);
        acc ^= __float_as_uint(v[0]) ^ __float_as_uint(v[1]) ^ __float_as_uint(v[2]) ^
               __float_as_uint(v[3]);
    }
    if (acc == 0x7FC0DEADu) *sink = acc;
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
    unsigned char* ws;
    size_t ws_bytes;
    u32 s_ws;
    u32 rowbytes;
    u32 chunk;
    u32 seg_full;
    u32 slots;
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

u32 ceil_div(u32 a, u32 b) { return (a + b - 1) / b; }

}  // namespace

extern "C" int sampler_create(tes_sampler** out, int device, int max_batch, int max_vocab,
                              unsigned flags) {
    if (!out) return TES_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    if (max_batch < 1 || max_vocab < 1 || max_vocab > (1 << 30) || device < 0)
        return TES_ERR_INVALID_ARGUMENT;
    if (flags & ~(TES_FLAG_FORCE_ROW_SELECT | TES_FLAG_TINY_BUFFER | TES_FLAG_STATS |
                  TES_FLAG_SMALL_SEGMENTS | TES_FLAG_NO_WAIT | TES_FLAG_ROW_TOPP))
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
    tes_sampler* s = new (std::nothrow) tes_sampler{};
    if (!s) return TES_ERR_OUT_OF_MEMORY;
    s->device = device;
    s->max_batch = max_batch;
    s->max_vocab = max_vocab;
    s->flags = flags;
    s->seg_full = (flags & TES_FLAG_SMALL_SEGMENTS) ? kSegVecSmall : kSegVecFull;
    // Two 512-thread workgroups fit on a compute unit (register bound).
    s->slots = 2u * (u32)(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1);
    // Exchange slots per row: enough for 16-byte rows of max_vocab; top-p-only
    // rows that need more segments (large scalar-path rows) use whole-row passes.
    s->s_ws = ceil_div(ceil_div((u32)max_vocab, 4), s->seg_full);
    if (s->s_ws < 1) s->s_ws = 1;
    if (s->s_ws > kMaxSegWs) s->s_ws = kMaxSegWs;
    size_t rb = (size_t)s->s_ws * (sizeof(PubC) + sizeof(PubF) + (size_t)kGSeg * sizeof(u64));
    if (rb < kSplitBytes) rb = kSplitBytes;  // parts of a split top-k or greedy row
    // One-workgroup top-p rows append up to one entry in eight of the row.
    if (rb < (size_t)max_vocab) rb = (size_t)max_vocab;
    rb = (rb + 255) & ~(size_t)255;
    s->rowbytes = (u32)rb;
    s->chunk = (u32)max_batch < kChunk ? (u32)max_batch : kChunk;
    // (and the fine histograms of a bf16 top-p-only row's segments)
    const size_t per_row =
        sizeof(RowState) + sizeof(Decision) + sizeof(XMax) + rb + (size_t)s->s_ws * sizeof(PubFF);
    const size_t budget_rows = kWsBudget / per_row;
    if (budget_rows < s->chunk) s->chunk = budget_rows < 1 ? 1u : (u32)budget_rows;
    s->ws_bytes = (size_t)s->chunk * per_row;
    DeviceGuard g(device);
    if (!g.ok) {
        delete s;
        return TES_ERR_NO_DEVICE;
    }
    if (hipMalloc(&s->ws, s->ws_bytes) != hipSuccess) {
        delete s;
        return TES_ERR_OUT_OF_MEMORY;
    }
    if (hipMemset(s->ws, 0, s->ws_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(s->ws);
        delete s;
        return TES_ERR_OUT_OF_MEMORY;
    }
    if (flags & TES_FLAG_STATS) {
        if (hipMalloc(&s->d_stats, sizeof(u32) * kStatWords * (size_t)max_batch) != hipSuccess) {
            (void)hipFree(s->ws);
            delete s;
            return TES_ERR_OUT_OF_MEMORY;
        }
    }
    *out = s;
    return TES_OK;
}

struct SlabOut {
    int32_t* index;
    float* renorm;
    int32_t* len;
    uint32_t* route;
    u32 cap;
};

namespace {
// The kernels of one launch (one chunk of rows) for row vectors of VEC entries.
template <int VEC, bool LG>
int launch_chunk(tes_sampler* s, const Params& p, hipStream_t st, u32 grid, u32 rows, u32 V,
                 u32 nvec, float* ro, const SlabOut* slab, size_t c0, const SpecArgs* spec) {
    if constexpr (LG) {
        hipLaunchKernelGGL(tes_rowmax_kernel<VEC>, dim3(p.xparts, rows), dim3(256), 0, st, p);
        if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
    }
    hipLaunchKernelGGL((tes_main_kernel<VEC, LG>), dim3(grid), dim3(kBlock), 0, st, p);
    if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
    const Decision* dec =
        reinterpret_cast<const Decision*>(s->ws + (size_t)s->chunk * sizeof(RowState));
    if (ro) {
        // About four vectors per thread, at most 64 workgroups per row unless
        // a workgroup's range would exceed kRenormSpan entries.
        const u32 gmin = ceil_div(nvec, kRenormSpan / (u32)VEC);
        u32 gx = ceil_div(nvec, 256 * 4) < 64 ? ceil_div(nvec, 256 * 4) : 64;
        gx = gx < gmin ? gmin : gx;
        hipLaunchKernelGGL((tes_renorm_kernel<VEC, LG>), dim3(gx, rows), dim3(256), 0, st, p, dec,
                           ro);
        if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
    }
    if constexpr (!LG && VEC != 8) {
        if (spec) {
            // The requests whose target rows this launch decided.
            const size_t n0 = c0 / spec->Lt;
            SpecArgs a = *spec;
            a.draft = spec->draft ? spec->draft + n0 * spec->L * (size_t)V : nullptr;
            a.tokens = spec->tokens ? spec->tokens + n0 * spec->L : nullptr;
            a.map = spec->map ? spec->map + n0 * (spec->L + 1) : nullptr;
            a.out = spec->out + n0 * (spec->L + 1);
            a.accept = spec->accept + n0;
            // Chunks per request: enough workgroups to fill the device (at
            // most eight, and none for rows of one round).
            const u32 nreq = rows / spec->Lt;
            u32 S = s->slots / nreq;
            S = S > 8 ? 8u : (S < 1 ? 1u : S);
            if (nvec <= 2 * kBlock) S = 1;
            hipLaunchKernelGGL(tes_verify_kernel<VEC>, dim3(nreq, S), dim3(kBlock), 0, st, p,
                               a);
            if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
        }
    }
    if (slab && !LG) {
        const size_t o = c0 * slab->cap;
        const unsigned char* lists =
            s->ws + (size_t)s->chunk * (sizeof(RowState) + sizeof(Decision) + sizeof(XMax));
        hipLaunchKernelGGL(tes_slab_kernel<VEC>, dim3(rows), dim3(kSlabThreads), 0, st, p.probs,
                           V, nvec, p.top_k, dec, lists, s->rowbytes, slab->cap, slab->index + o,
                           slab->renorm + o, slab->len + c0,
                           slab->route ? slab->route + c0 : nullptr);
        if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
    }
    return TES_OK;
}

// probs holds fp32 entries, or bf16 entries when bf16 is set, or fp32 logits
// when logits is set (with the nullable per-row temperature; min_p, nullable,
// applies to both kinds of rows).
// With spec (speculative verification), B counts target rows (Lt per
// request), launches take whole requests, and the verification kernel
// follows each launch; out_tokens is not used (the outputs are spec's).
int sample_impl(tes_sampler* s, const void* probs, bool bf16, int B, int V, const int32_t* top_k,
                const float* top_p, uint64_t seed, uint64_t offset, int32_t* out_tokens,
                float* renorm_out, const SlabOut* slab, void* stream, bool logits = false,
                const float* temperature = nullptr, const float* min_p = nullptr,
                const SpecArgs* spec = nullptr) {
    if (!s || B < 0 || V < 1) return TES_ERR_INVALID_ARGUMENT;
    if (B > s->max_batch || V > s->max_vocab) return TES_ERR_TOO_LARGE;
    if (B == 0) return TES_OK;
    if (!probs || !top_k || !top_p || (!out_tokens && !spec)) return TES_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)probs & 3) || ((uintptr_t)top_k & 3) || ((uintptr_t)top_p & 3) ||
        ((uintptr_t)out_tokens & 3) || ((uintptr_t)renorm_out & 3) ||
        ((uintptr_t)temperature & 3) || ((uintptr_t)min_p & 3))
        return TES_ERR_INVALID_ARGUMENT;
    if (logits && (bf16 || slab)) return TES_ERR_INVALID_ARGUMENT;
    if (spec && (logits || bf16 || slab)) return TES_ERR_INVALID_ARGUMENT;
    // Row vectors: eight bf16 entries (bf16 rows must allow them), four fp32
    // entries when the rows and renorm_out allow 16-byte access, else one.
    const bool aligned16 = (((uintptr_t)probs & 15) == 0) && (((uintptr_t)renorm_out & 15) == 0);
    if (bf16 && (V % 8 != 0 || !aligned16)) return TES_ERR_INVALID_ARGUMENT;
    const int vec = bf16 ? 8 : ((V % 4 == 0) && aligned16 ? 4 : 1);
    const size_t entry_bytes = bf16 ? 2 : 4;
    DeviceGuard g(s->device);
    if (!g.ok) return TES_ERR_LAUNCH;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const u32 nvec = (u32)V / (u32)vec;
    const u32 seg = vec == 8 ? s->seg_full / 2 : s->seg_full;  // vectors per segment
    const u32 s_full = ceil_div(nvec, seg);
    // Rows per launch (whole requests under spec).
    const u32 step = spec ? (s->chunk / spec->Lt) * spec->Lt : s->chunk;
    if (step == 0) return TES_ERR_TOO_LARGE;
    for (int c0 = 0; c0 < B; c0 += (int)step) {
        const u32 rows = (u32)(B - c0) < step ? (u32)(B - c0) : step;
        Params p;
        p.probs = reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(probs) +
                                                 (size_t)c0 * V * entry_bytes);
        p.top_k = top_k + c0;
        p.top_p = top_p + c0;
        p.temperature = temperature ? temperature + c0 : nullptr;
        p.min_p = min_p ? min_p + c0 : nullptr;
        p.out_tokens = out_tokens ? out_tokens + c0 : nullptr;
        p.stats = (s->flags & TES_FLAG_STATS) ? s->d_stats : nullptr;
        p.ws = s->ws;
        p.seed = seed;
        p.offset = offset;
        p.V = (u32)V;
        p.nvec = nvec;
        p.rows = rows;
        p.row_base = (u32)c0;
        p.seg_vec_full = seg;
        p.s_ws = s->s_ws;
        p.rowbytes = s->rowbytes;
        p.chunk = s->chunk;
        p.flags = s->flags;
        if (renorm_out || slab) p.flags |= kFlagList;
        if (slab) p.flags |= kFlagSupport;
        // Top-k and greedy rows may be split into up to kMaxSplit parts of at
        // least kMinPartVec vectors (the kernel splits only when every part
        // is resident at once).
        const u32 by_len = nvec / kMinPartVec;
        p.split = s->rowbytes >= kSplitBytes ? (by_len < kMaxSplit ? (by_len < 1 ? 1u : by_len) : kMaxSplit)
                                             : 1u;
        p.slots = s->slots;
        // Logit rows: parts per row of the row-maximum prologue (enough
        // workgroups to fill the device for small batches).
        {
            const u32 want = ceil_div(2 * s->slots, rows);
            const u32 by_len = ceil_div(nvec, 4 * 256);
            u32 xp = want < kXParts ? want : kXParts;
            xp = xp < by_len ? xp : by_len;
            p.xparts = xp < 1 ? 1u : xp;
        }
        if (p.stats) {
            const u32 nw = kStatWords * rows;
            hipLaunchKernelGGL(tes_clear_kernel, dim3(ceil_div(nw, 256) < 64 ? ceil_div(nw, 256) : 64),
                               dim3(256), 0, st, p.stats + (size_t)kStatWords * c0, nw);
            if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
        }
        // Enough blocks for every row to be top-p-only; the kernel knows the
        // actual mix, and blocks beyond the last item return at once.
        // Split rows occur only when every item is resident, i.e. within
        // the slots.  Segmented rows too: a launch whose items would exceed
        // the slots decides its top-p-only rows one item each, so there are
        // never more than max(rows, slots) items.
        const u32 per_row = s_full <= s->s_ws ? s_full : 1u;
        const u32 split_items = rows * p.split < s->slots ? rows * p.split : s->slots;
        const u32 g_all = rows * per_row > split_items ? rows * per_row : split_items;
        const u32 g_cap = rows > s->slots ? rows : s->slots;
        const u32 grid = g_all < g_cap ? g_all : g_cap;
        float* ro = renorm_out ? renorm_out + (size_t)c0 * V : nullptr;
        const int rc =
            logits ? (vec == 4 ? launch_chunk<4, true>(s, p, st, grid, rows, (u32)V, nvec, ro, slab,
                                                       c0, spec)
                               : launch_chunk<1, true>(s, p, st, grid, rows, (u32)V, nvec, ro, slab,
                                                       c0, spec))
            : vec == 8 ? launch_chunk<8, false>(s, p, st, grid, rows, (u32)V, nvec, ro, slab, c0, spec)
            : vec == 4 ? launch_chunk<4, false>(s, p, st, grid, rows, (u32)V, nvec, ro, slab, c0, spec)
                       : launch_chunk<1, false>(s, p, st, grid, rows, (u32)V, nvec, ro, slab, c0, spec);
        if (rc != TES_OK) return rc;
    }
    return TES_OK;
}
}  // namespace

extern "C" int topk_topp_sample(tes_sampler* s, const float* probs, int B, int V,
                                const int32_t* top_k, const float* top_p, uint64_t seed,
                                uint64_t offset, int32_t* out_tokens, float* renorm_out,
                                void* stream) {
    return sample_impl(s, probs, false, B, V, top_k, top_p, seed, offset, out_tokens, renorm_out,
                       nullptr, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free entry point
// ---------------------------------------------------------------------------
// topk_topp_sample_noalloc keeps its workspace (row states, decisions and the
// per-row exchange areas of up to kNoAllocRows rows, laid out exactly as a
// handle's workspace) in one statically sized device array, so that a call
// allocates nothing.  Its size is fixed by the largest vocabulary it serves;
// batches of more rows run as several launches.
namespace {
constexpr u32 kNoAllocRows = 256;
constexpr u32 kNoAllocMaxVocab = 1u << 18;
constexpr u32 kNoAllocSegWs = (kNoAllocMaxVocab / 4 + kSegVecFull - 1) / kSegVecFull;
constexpr size_t kNoAllocTopP =
    (size_t)kNoAllocSegWs * (sizeof(PubC) + sizeof(PubF) + (size_t)kGSeg * sizeof(u64));
constexpr size_t kNoAllocRowBytes =
    ((kNoAllocTopP > kSplitBytes ? kNoAllocTopP : kSplitBytes) + 255) & ~(size_t)255;
constexpr size_t kScratchBytes =
    (size_t)kNoAllocRows * (sizeof(RowState) + sizeof(Decision) + sizeof(XMax) + kNoAllocRowBytes);
static_assert(kNoAllocRows * sizeof(RowState) % 4 == 0, "row states clear as words");
static_assert(kScratchBytes <= (40u << 20), "the scratch array stays modest");
}  // namespace

// One copy per GPU the library runs on, held until the process ends.  Host
// code never uses this name as an address: the device address of each GPU's
// copy comes from hipGetSymbolAddress (see noalloc_device).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
struct NoAllocDevice {
    unsigned char* ptr;  // device address of this GPU's scratch array (null: not set up)
    u32 slots;           // resident workgroups
    bool clean;          // its row states were cleared by an executed (not captured) call
};
constexpr int kNoAllocDevices = 64;
std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kNoAllocDevices];

// Sets up device `dev` (current) on its first call: checks the architecture,
// takes the scratch array's device address and clears its row states with a
// kernel on `st` (row states must start at zero; the sampler leaves them at
// zero after every row).  A clear recorded into a graph under capture does
// not count: the next call that is not captured clears again.
int noalloc_device(int dev, hipStream_t st, NoAllocDevice& out) {
    if (dev < 0 || dev >= kNoAllocDevices) return TES_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    NoAllocDevice& e = g_noalloc[dev];
    if (!e.ptr) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TES_ERR_NO_DEVICE;
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return TES_ERR_UNSUPPORTED_DEVICE;
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return TES_ERR_LAUNCH;
        }
        e.ptr = static_cast<unsigned char*>(ptr);
        e.slots = 2u * (u32)(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1);
        e.clean = false;
    }
    if (!e.clean) {
        const u32 nw = (u32)(kNoAllocRows * sizeof(RowState) / 4);
        hipLaunchKernelGGL(tes_clear_kernel, dim3(ceil_div(nw, 256)), dim3(256), 0, st,
                           reinterpret_cast<u32*>(e.ptr), nw);
        if (hipGetLastError() != hipSuccess) return TES_ERR_LAUNCH;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
            e.clean = true;
        else
            (void)hipGetLastError();
    }
    out = e;
    return TES_OK;
}
}  // namespace

extern "C" int topk_topp_sample_noalloc(const float* probs, int B, int V, const int32_t* top_k,
                                        const float* top_p, uint64_t seed, uint64_t offset,
                                        int32_t* out_tokens, float* renorm_out, void* stream) {
    if (B < 0 || V < 1) return TES_ERR_INVALID_ARGUMENT;
    if ((u32)V > kNoAllocMaxVocab) return TES_ERR_TOO_LARGE;
    if (B == 0) return TES_OK;
    // Argument errors are reported before the device is touched.
    if (!probs || !top_k || !top_p || !out_tokens) return TES_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)probs & 3) || ((uintptr_t)top_k & 3) || ((uintptr_t)top_p & 3) ||
        ((uintptr_t)out_tokens & 3) || ((uintptr_t)renorm_out & 3))
        return TES_ERR_INVALID_ARGUMENT;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return TES_ERR_NO_DEVICE;
    }
    NoAllocDevice d{};
    const int rc = noalloc_device(dev, reinterpret_cast<hipStream_t>(stream), d);
    if (rc != TES_OK) return rc;
    // A handle-shaped view of the scratch array (nothing is allocated).
    tes_sampler view{};
    view.device = dev;
    view.max_batch = INT_MAX;
    view.max_vocab = (int)kNoAllocMaxVocab;
    view.flags = 0;
    view.ws = d.ptr;
    view.ws_bytes = kScratchBytes;
    view.s_ws = kNoAllocSegWs;
    view.rowbytes = (u32)kNoAllocRowBytes;
    view.chunk = kNoAllocRows;
    view.seg_full = kSegVecFull;
    view.slots = d.slots;
    view.d_stats = nullptr;
    return sample_impl(&view, probs, false, B, V, top_k, top_p, seed, offset, out_tokens,
                       renorm_out, nullptr, stream);
}

extern "C" int topk_topp_sample_logits(tes_sampler* s, const float* logits, int B, int V,
                                       const int32_t* top_k, const float* top_p,
                                       const float* temperature, const float* min_p,
                                       uint64_t seed, uint64_t offset, int32_t* out_tokens,
                                       float* renorm_out, void* stream) {
    return sample_impl(s, logits, false, B, V, top_k, top_p, seed, offset, out_tokens, renorm_out,
                       nullptr, stream, true, temperature, min_p);
}

extern "C" int spec_verify_sample(tes_sampler* s, const float* target_probs, int N, int Lt,
                                  int V, const int32_t* top_k, const float* top_p,
                                  const float* draft_probs, int L, const int32_t* draft_tokens,
                                  const int32_t* target_map, uint64_t seed, uint64_t offset,
                                  int32_t* out_tokens, int32_t* accept_len, void* stream) {
    if (!s || N < 0 || Lt < 1 || V < 1 || L < 0 || L > 63) return TES_ERR_INVALID_ARGUMENT;
    if (!target_map && Lt < L + 1) return TES_ERR_INVALID_ARGUMENT;
    if ((int64_t)N * Lt > s->max_batch || V > s->max_vocab) return TES_ERR_TOO_LARGE;
    if (N == 0) return TES_OK;
    if (!out_tokens || !accept_len || (L > 0 && (!draft_probs || !draft_tokens)))
        return TES_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)out_tokens & 3) || ((uintptr_t)accept_len & 3) ||
        ((uintptr_t)draft_tokens & 3) || ((uintptr_t)target_map & 3))
        return TES_ERR_INVALID_ARGUMENT;
    // The verification reads draft rows with the target rows' vector width.
    const bool t16 = ((uintptr_t)target_probs & 15) == 0 && V % 4 == 0;
    const bool d16 = ((uintptr_t)draft_probs & 15) == 0;
    if (L > 0 && t16 && !d16) return TES_ERR_INVALID_ARGUMENT;
    if (L > 0 && ((uintptr_t)draft_probs & 3)) return TES_ERR_INVALID_ARGUMENT;
    SpecArgs a{draft_probs, draft_tokens, target_map, out_tokens, accept_len, (u32)L, (u32)Lt};
    return sample_impl(s, target_probs, false, N * Lt, V, top_k, top_p, seed, offset, nullptr,
                       nullptr, nullptr, stream, false, nullptr, nullptr, &a);
}

extern "C" int topk_topp_sample_bf16(tes_sampler* s, const uint16_t* probs, int B, int V,
                                     const int32_t* top_k, const float* top_p, uint64_t seed,
                                     uint64_t offset, int32_t* out_tokens, float* renorm_out,
                                     void* stream) {
    return sample_impl(s, probs, true, B, V, top_k, top_p, seed, offset, out_tokens, renorm_out,
                       nullptr, stream);
}

extern "C" int topk_topp_sample_slab(tes_sampler* s, const float* probs, int B, int V,
                                     const int32_t* top_k, const float* top_p, uint64_t seed,
                                     uint64_t offset, int32_t* out_tokens, float* renorm_out,
                                     int32_t* slab_index, float* slab_renorm, int slab_cap,
                                     int32_t* slab_len, uint32_t* route, void* stream) {
    if (B > 0 && (!slab_index || !slab_renorm || !slab_len)) return TES_ERR_INVALID_ARGUMENT;
    if (slab_cap < 1 || slab_cap > (int)kSlabExportMax) return TES_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)slab_index & 3) || ((uintptr_t)slab_renorm & 3) || ((uintptr_t)slab_len & 3) ||
        ((uintptr_t)route & 3))
        return TES_ERR_INVALID_ARGUMENT;
    const SlabOut slab{slab_index, slab_renorm, slab_len, route, (u32)slab_cap};
    return sample_impl(s, probs, false, B, V, top_k, top_p, seed, offset, out_tokens, renorm_out,
                       &slab, stream);
}

extern "C" int sampler_route(tes_sampler* s, int B, int V, const int32_t* top_k_host,
                             uint32_t* route_host) {
    if (!s || B < 0 || V < 1 || (B > 0 && (!top_k_host || !route_host)))
        return TES_ERR_INVALID_ARGUMENT;
    if (B > s->max_batch || V > s->max_vocab) return TES_ERR_TOO_LARGE;
    // Rows are 16-byte streamed when V % 4 == 0 (with an aligned base); the
    // segment count of a top-p-only row follows from that.
    const u32 nvec = (V % 4 == 0) ? (u32)V / 4 : (u32)V;
    const u32 s_full = ceil_div(nvec, s->seg_full);
    for (int b = 0; b < B; ++b) {
        const int32_t k = top_k_host[b];
        const u32 k_eff = (k <= 0 || k >= V) ? (u32)V : (u32)k;
        u32 path;
        if (s->flags & TES_FLAG_FORCE_ROW_SELECT) path = kPathWhole;
        else if (k_eff == 1) path = kPathGreedy;
        else if (k_eff <= kSlabMaxK) path = kPathSlab;
        else if (k_eff == (u32)V && s_full <= s->s_ws) path = kPathFull;
        else path = kPathWhole;
        route_host[b] = path;
    }
    return TES_OK;
}

extern "C" int sampler_destroy(tes_sampler* s) {
    if (!s) return TES_OK;
    {
        DeviceGuard g(s->device);
        if (s->ws) (void)hipFree(s->ws);
        if (s->d_stats) (void)hipFree(s->d_stats);
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

extern "C" int sampler_read_probe(const void* data, uint64_t bytes, uint32_t* sink, int device,
                                  void* stream) {
    if (!data || !sink || device < 0 || ((uintptr_t)data & 15) || (bytes & 15) ||
        ((uintptr_t)sink & 3))
        return TES_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return TES_OK;
    DeviceGuard g(device);
    if (!g.ok) return TES_ERR_LAUNCH;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const u64 nvec = bytes / 16;
    const u64 want = (nvec + 256 * 8 - 1) / (256 * 8);
    const u32 grid = want < 8192 ? (u32)(want < 1 ? 1 : want) : 8192u;
    hipLaunchKernelGGL(tes_read_kernel, dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const f4*>(data), nvec, sink);
    return hipGetLastError() == hipSuccess ? TES_OK : TES_ERR_LAUNCH;
}

extern "C" int sampler_get_stats(tes_sampler* s, uint32_t* host_out, int B) {
    if (!s || !host_out || B < 0 || B > s->max_batch) return TES_ERR_INVALID_ARGUMENT;
    if (!s->d_stats) return TES_ERR_INVALID_ARGUMENT;
    DeviceGuard g(s->device);
    if (!g.ok) return TES_ERR_LAUNCH;
    if (hipDeviceSynchronize() != hipSuccess) return TES_ERR_LAUNCH;
    if (hipMemcpy(host_out, s->d_stats, sizeof(u32) * kStatWords * (size_t)B,
                  hipMemcpyDeviceToHost) != hipSuccess)
        return TES_ERR_LAUNCH;
    return TES_OK;
}
