/*
 * tes_sampler.h -- C ABI of the MI355X (gfx950) exact top-k -> top-p sampler.
 *
 * Operation (FlashInfer "cake_sampling" documentation page, section
 * "Semantics", and its description of the sparse top-p stage): for every row
 * b of a [B][V] fp32 probability matrix,
 *   1. sanitise: NaN, negative and -0.0 entries count as +0 and are never
 *      sampled; +inf is kept;
 *   2. support S = the first k_eff entries of lexsort(-prob, index), i.e. a
 *      stable descending sort with ties going to the lower vocabulary index;
 *      k_eff = V when top_k[b] <= 0 or top_k[b] >= V, else top_k[b];
 *   3. if S holds m > 0 entries equal to +inf, exactly those are kept with
 *      weight 1/m and the draw is uniform among them;
 *   4. otherwise masses q = floor(min(prob, 1) * 2^32) (exact integers) and
 *      M_k = sum over S.  If M_k = 0 the token is the smallest vocabulary index
 *      in S and the renormalised row is all zero;
 *   5. top-p on exact 64-bit fixed-point prefix sums: P = round-half-even(
 *      top_p[b] * 2^24) clamped to [1, 2^24] (NaN or <= 0 gives 1, >= 1 gives
 *      2^24); sorted position j is kept while its exclusive prefix mass is
 *      below ceil(P * M_k / 2^24).  This is the shortest prefix holding at
 *      least top_p of the top-k mass (the nucleus of the SonicSampler paper,
 *      eq. (10), taken relative to the top-k mass);
 *   6. one inverse-CDF draw per row: u = x0 | x1 << 32 of Philox4x32-10
 *      (Salmon et al., SC'11) with key (seed lo, seed hi) and counter
 *      (offset lo, offset hi, b lo, b hi); t = floor(u * M_p / 2^64) with M_p
 *      the kept mass; token = first kept position whose inclusive prefix mass
 *      exceeds t;
 *   7. optional renormalised output: renorm_out[b][i] = fp32(q_i / M_p) for kept
 *      i (1/m for kept +inf entries), 0 elsewhere.
 * Every decision is integer arithmetic, so results are bitwise reproducible
 * across launches, streams and internal paths.
 *
 * Status codes: 0 on success, a negative TES_ERR_* value on failure.  Nothing
 * aborts or throws across this interface.  Probability values are never an
 * error (NaN, negatives, zero rows and out-of-range top_k / top_p follow the
 * rules above and every output is finite).
 */
#ifndef TES_SAMPLER_H
#define TES_SAMPLER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TES_OK 0
#define TES_ERR_INVALID_ARGUMENT (-1) /* bad handle, pointer, size or alignment */
#define TES_ERR_NO_DEVICE (-2)        /* no HIP device, or device index out of range */
#define TES_ERR_UNSUPPORTED_DEVICE (-3) /* device is not gfx950 */
#define TES_ERR_OUT_OF_MEMORY (-4)    /* host or device allocation failed at create */
#define TES_ERR_LAUNCH (-5)           /* HIP runtime error while enqueueing */
#define TES_ERR_TOO_LARGE (-6)        /* B or V above the limits given at create */

/* Flags for sampler_create.  They select internal paths for testing; none of
 * them changes any output. */
#define TES_FLAG_NONE 0u
/* Resolve every row with the multi-pass whole-row select instead of the
 * single-read candidate buffer. */
#define TES_FLAG_FORCE_ROW_SELECT 1u
/* Compact the top-k candidate buffer whenever it holds more than k entries,
 * and shrink the gather capacities of the other paths, so that compaction
 * and the multi-pass fallback run on ordinary inputs. */
#define TES_FLAG_TINY_BUFFER 2u
/* Record per-row path statistics (see sampler_get_stats). */
#define TES_FLAG_STATS 4u
/* Cut top-p-only rows into segments of 4096 floats instead of 32768, so that
 * the cross-segment exchanges run on small vocabularies too. */
#define TES_FLAG_SMALL_SEGMENTS 8u
/* Make every bounded wait of the cross-workgroup exchanges report a timeout
 * without polling, so that a top-p-only row cut into several segments takes
 * the path that a timed-out exchange takes (its whole-row passes decide it).
 * Outputs are unchanged; only the path differs. */
#define TES_FLAG_NO_WAIT 16u
/* Decide every top-p-only row by one workgroup in one pass over the row
 * (plus a second visit of its first sixteenth), with no exchange between
 * workgroups: the path taken anyway when a launch holds more top-p-only
 * segments than the device keeps resident workgroups. */
#define TES_FLAG_ROW_TOPP 32u

typedef struct tes_sampler tes_sampler;

/* Create a sampler bound to HIP device `device`.
 *   out        receives the handle (host pointer; must not be NULL).
 *   max_batch  largest B any later call may pass (>= 1).
 *   max_vocab  largest V any later call may pass (1 .. 2^30).
 *   flags      TES_FLAG_* bits.
 * The handle owns its device workspace (at most about 512 MiB; batches of
 * more rows than it holds run as several launches), allocated here and
 * released by sampler_destroy.  Returns TES_ERR_NO_DEVICE when no GPU is present,
 * TES_ERR_UNSUPPORTED_DEVICE when the device is not gfx950. */
int sampler_create(tes_sampler **out, int device, int max_batch, int max_vocab,
                   unsigned flags);

/* Sample one token per row; asynchronous on `stream`.
 *   probs       device, fp32 [B][V] row-major, contiguous, 4-byte aligned
 *               (16-byte alignment and V % 4 == 0 enable 16-byte loads);
 *               read only.
 *   B, V        batch rows (0 .. max_batch; B = 0 is a no-op) and vocabulary
 *               size (1 .. max_vocab).
 *   top_k       device, int32 [B]; <= 0 or >= V disables top-k.
 *   top_p       device, fp32 [B]; clamped as described above.
 *   seed,offset Philox key and 128-bit-block offset; row b uses counter
 *               (offset, b).  Advance offset by at least 1 between calls
 *               that must draw independently.
 *   out_tokens  device, int32 [B]; receives the sampled vocabulary index.
 *   renorm_out  device, fp32 [B][V] or NULL; when given, every entry of every
 *               row is written (dense, vocabulary order).
 *   stream      hipStream_t (NULL = default stream) on the sampler's device.
 * All device buffers are owned by the caller and must stay valid until the
 * enqueued work completes; outputs must not alias probs.  No allocation and
 * no host synchronisation happen inside the call.  One handle must not be
 * used from two streams concurrently. */
int topk_topp_sample(tes_sampler *s, const float *probs, int B, int V, const int32_t *top_k,
                     const float *top_p, uint64_t seed, uint64_t offset, int32_t *out_tokens,
                     float *renorm_out, void *stream);

/* Sampling from fp32 logit rows with a per-row temperature and a min-p floor
 * (SonicSampler paper, appendix C.1 "Temperature", eq. (8), and appendix C.2
 * "Min-p", eqs. (11)-(12)).  Each row becomes fp32 weights: with M the row
 * maximum (NaN counts as -inf) and r = fp32(fp64(1 / tau)), an entry equal to
 * M weighs 1 and any other E((x - M) * r), E an fp32 exponential evaluated
 * by a fixed sequence of correctly rounded fp32 operations (Cody-Waite
 * reduction, degree-7 Taylor polynomial; within one ulp of exp, 0 below
 * 2^-125), so the weights are bit-reproducible; tau NaN or <= 0 is the
 * tau -> 0 limit (1 on every maximum, 0 elsewhere), tau = +inf weighs every
 * finite entry 1; rows with a +inf logit weigh their +inf entries +inf (the
 * +inf rule), rows of only -inf / NaN weigh everything 0.  The weights are
 * softmax(x / tau) up to one scale factor, which every step cancels; the row
 * is then sampled by steps 1-7 above, with min-p after top-p: the support
 * entries with mass q < ceil(theta * q_max) (q_max the largest mass) are
 * dropped from the kept prefix.  renorm_out holds the final probabilities.
 *   logits       device, fp32 [B][V] row-major, contiguous, 4-byte aligned
 *                (16-byte alignment and V % 4 == 0 enable 16-byte loads).
 *   temperature  device, fp32 [B], or NULL (1 on every row).
 *   min_p        device, fp32 [B], or NULL (off); theta NaN or <= 0 is off,
 *                theta > 1 counts as 1.
 * Every other argument, the ownership rules and the status codes are those
 * of topk_topp_sample.  One extra read of the rows (their maxima) precedes
 * the sampling kernel. */
int topk_topp_sample_logits(tes_sampler *s, const float *logits, int B, int V,
                            const int32_t *top_k, const float *top_p, const float *temperature,
                            const float *min_p, uint64_t seed, uint64_t offset,
                            int32_t *out_tokens, float *renorm_out, void *stream);

/* Speculative verification on the sampled target rows (SonicSampler paper,
 * appendix C.4 "Speculative Verification", eqs. (15)-(16), and its
 * "Draft-to-Target Mapping").  N requests; request n proposed L draft tokens
 * d_l from draft distributions q_l and owns Lt target rows.  Draft position
 * l (and the bonus position L) reads target row g = n * Lt + pi(l), pi =
 * target_map[n][l] (the identity when target_map is NULL).  Each target row
 * is first sampled as by topk_topp_sample (its own top_k / top_p; its final
 * distribution p_g and its own token, drawn with Philox words 0-1 of row g).
 * Then, for l = 0, 1, ...:
 *   accept d_l  iff  u_a * q_l(d_l) <= p_g(d_l), compared exactly, with
 *               u_a = (word2 | word3 << 32) / 2^64 of row g's Philox block and
 *               q_l(x) = floor(min(y_x, 1) * 2^32) / 2^32 of the sanitised
 *               draft probability y_x (the draft row as given);
 *   at the first rejection, the correction token is drawn from
 *               max(0, p_g - q_l) normalised, by integer inverse CDF in
 *               vocabulary order with row g's own 64-bit uniform (its own
 *               token when p_g <= q_l everywhere), and the request stops;
 *   if every draft is accepted, the bonus token is row pi(L)'s own token.
 *   target_probs  device, fp32 [N * Lt][V], as for topk_topp_sample.
 *   top_k, top_p  device, [N * Lt], per target row.
 *   draft_probs   device, fp32 [N][L][V]; 16-byte aligned when target_probs is
 *                 16-byte aligned and V % 4 == 0.  NULL when L = 0.
 *   draft_tokens  device, int32 [N][L].  NULL when L = 0.
 *   target_map    device, int32 [N][L + 1], or NULL (then Lt >= L + 1).
 *   out_tokens    device, int32 [N][L + 1]: the accepted drafts, then the
 *                 correction or the bonus token, then -1.
 *   accept_len    device, int32 [N]: the number of accepted drafts (0 .. L);
 *                 -1 (and all tokens -1) for a request whose map entries lie
 *                 outside [0, Lt) or whose draft tokens lie outside [0, V).
 * L is 0 .. 63; N * Lt <= max_batch.  Status codes as for topk_topp_sample. */
int spec_verify_sample(tes_sampler *s, const float *target_probs, int N, int Lt, int V,
                       const int32_t *top_k, const float *top_p, const float *draft_probs, int L,
                       const int32_t *draft_tokens, const int32_t *target_map, uint64_t seed,
                       uint64_t offset, int32_t *out_tokens, int32_t *accept_len, void *stream);

/* topk_topp_sample for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same sampling, outputs and argument rules, with no handle.
 * Its workspace is one statically sized device array of the library (about
 * 32 MiB per GPU, taken when the library is loaded and held until the process
 * ends); the call allocates nothing.
 *   device      the current HIP device (hipGetDevice) when the call is made.
 *   V           1 .. 262144 (TES_ERR_TOO_LARGE above); any B >= 0 (batches
 *               of more than 256 rows run as several launches).
 *   stream      hipStream_t on the current device.
 * The first call on a device sets up that device (architecture check, the
 * array's device address) and clears the array's row states with a kernel
 * on `stream`.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Returns TES_ERR_NO_DEVICE without a current
 * device, TES_ERR_UNSUPPORTED_DEVICE when it is not gfx950, otherwise the
 * statuses of topk_topp_sample. */
int topk_topp_sample_noalloc(const float *probs, int B, int V, const int32_t *top_k,
                             const float *top_p, uint64_t seed, uint64_t offset,
                             int32_t *out_tokens, float *renorm_out, void *stream);

/* topk_topp_sample over bfloat16 probability rows (the 16-bit format whose
 * ordered encoding the SonicSampler page builds its keys from, section 3.4
 * "Numerical Lexicographic Encoding"; its input there is bf16 logits).
 * Each entry means exactly its widening to fp32 (the 16 bits become the
 * upper half of an fp32 word); after that every step -- support, cutoff,
 * draw, renormalisation -- is the fp32 method, so the tokens equal those of
 * topk_topp_sample on the widened rows.  Half the bytes are read.
 *   probs       device, bf16 bit patterns [B][V] row-major, contiguous;
 *               16-byte aligned and V % 8 == 0 (TES_ERR_INVALID_ARGUMENT
 *               otherwise).
 *   renorm_out  device, fp32 [B][V] or NULL, 16-byte aligned when given.
 * Every other argument, the ownership rules and the status codes are those
 * of topk_topp_sample. */
int topk_topp_sample_bf16(tes_sampler *s, const uint16_t *probs, int B, int V,
                          const int32_t *top_k, const float *top_p, uint64_t seed,
                          uint64_t offset, int32_t *out_tokens, float *renorm_out, void *stream);

/* topk_topp_sample plus the slab export: the same sampling (same arguments,
 * same outputs), and for every row whose support holds at most slab_cap
 * entries, the support in its sorted order -- descending probability,
 * ascending vocabulary index, the order in which the FlashInfer
 * "cake_sampling" page (section "Semantics") emits its workspace slab and
 * renormalised output -- with the renormalised weight of each entry.
 *   slab_index   device, int32 [B][slab_cap]: row b's support indices in
 *                sorted order at [b][0, len), -1 after them.
 *   slab_renorm  device, fp32 [B][slab_cap]: the renormalised weight of
 *                slab_index[b][j] (exactly the renorm_out value at that
 *                index: q / M_p for kept entries, 1/m for kept +inf entries,
 *                0 for support entries past the top-p cut and for zero-mass
 *                rows), 0 after len.
 *   slab_cap     1 .. 1024.
 *   slab_len     device, int32 [B]: the support size k_eff, or -1 when it
 *                exceeds slab_cap (then the row's slab is all -1 / 0).
 *   route        device, uint32 [B] or NULL: the path that decided each row
 *                (the codes of sampler_get_stats word [0]).
 * The export reads every row once more (one extra pass over probs).  Errors
 * as for topk_topp_sample, plus TES_ERR_INVALID_ARGUMENT for a slab_cap out
 * of range or null / misaligned slab pointers. */
int topk_topp_sample_slab(tes_sampler *s, const float *probs, int B, int V,
                          const int32_t *top_k, const float *top_p, uint64_t seed,
                          uint64_t offset, int32_t *out_tokens, float *renorm_out,
                          int32_t *slab_index, float *slab_renorm, int slab_cap,
                          int32_t *slab_len, uint32_t *route, void *stream);

/* The path each row will take, from top_k in host memory, without launching
 * anything (the role of the cake_sampling page's route report): 4 greedy
 * (k_eff = 1), 0 top-k streaming (k_eff <= 1024), 1 top-p-only (k_eff = V),
 * 3 whole-row passes (1024 < k_eff < V, or forced by the flags).  Data can
 * still send a row to a fallback (codes 2 and 5 of sampler_get_stats); the
 * route output of topk_topp_sample_slab reports the path actually taken.
 *   top_k_host  host, int32 [B];  route_host  host, uint32 [B]. */
int sampler_route(tes_sampler *s, int B, int V, const int32_t *top_k_host,
                  uint32_t *route_host);

/* Release the handle and its workspace.  NULL is accepted. */
int sampler_destroy(tes_sampler *s);

/* Static English description of a status code. */
const char *sampler_status_string(int status);

/* Copy per-row path statistics of the last call (handle created with
 * TES_FLAG_STATS) to host memory: 16 uint32 per row =
 *   [0] path: 0 top-k row (k <= 1024) resolved from its candidate buffer,
 *       1 top-p-only row resolved from exchanged histograms and gathered bins,
 *       2 top-p-only row that fell back to whole-row passes,
 *       3 row resolved by whole-row passes (1024 < k < V, or forced),
 *       4 greedy row (k = 1),
 *       5 top-k row decided by one compacting pass over the whole row
 *         (its sampled threshold could not decide it: too few sampled
 *         entries with a mass, or a run of equal values that overflowed
 *         the candidate buffer),
 *       6 top-p-only row decided by one workgroup (TES_FLAG_ROW_TOPP, or a
 *         launch with more top-p-only segments than resident workgroups);
 *   [1] kind: 0 normal, 1 +inf row, 2 zero-mass row;
 *   [2] segments the row was cut into;
 *   [3] candidate-buffer compactions (paths 0 and 5) or passes over the row
 *       (path 3);
 *   [4] entries gathered for the final selects (paths 0, 1, 2);
 *   [5] device wall clock when the row was resolved (low 32 bits);
 *   [6] 0xFFFFFFFF minus the earliest wall clock at which a segment of the
 *       row started;
 *   [7] why a row left its fast path (bits): 1 first exchange timed out,
 *       2 the draw spans more coarse bins than are exchanged (their count in
 *       bits 8..15), 4 second exchange timed out (fp32 rows; bf16 rows
 *       have no second exchange), 8 inconsistent fine bins,
 *       16 a segment gathered too many entries, 32 too many in total (these
 *       for top-p-only rows), 64 a top-k row's binned finish needed a sort;
 *       path 6: 1 << 16 its appended entries overflowed, 1 << 17 the
 *       boundary's bin was not appended whole, 1 << 18 nor the draw's,
 *       1 << 19 it fell back to whole-row passes (path 2);
 *   [8..15] wall-clock ticks spent in successive phases, summed over the
 *       row's workgroups: greedy [8] whole item; top-k [8] streaming,
 *       [9] the finish, [11] the sampled first part, [13] the rest of the
 *       stream, [14] and [15] the padding and the sort when the finish
 *       sorts; top-p-only [8] loads and histogram, [9] first exchange,
 *       [10] its analysis and the second publication, [11] second exchange
 *       (bf16 rows: nothing, their fine histograms went with the first),
 *       [12] gather and arrival, [13] the last segment's finish, [14] its
 *       loads, [15] its boundary select; other words 0.  Exception: with
 *       renorm_out, [10] of a top-k or greedy row holds the number of kept
 *       entries it recorded (renorm_out's row is then written without
 *       reading the row again); with the slab export, the number of positive
 *       support entries it recorded (the slab is then sorted from them when
 *       they are the whole support).
 * The wall clock is the device's constant 100 MHz counter.  Synchronises the
 * device.  `host_out` holds 16 * B uint32. */
int sampler_get_stats(tes_sampler *s, uint32_t *host_out, int B);

/* Reference measurement, not part of sampling: reads `bytes` bytes of device
 * memory at `data` once with coalesced 16-byte loads (the access pattern of
 * the sampler's row stream, with nothing computed) on `stream`, on HIP device
 * `device`.  Timing it over the same bytes as a sampler call gives the plain
 * read time of the device, the practical floor of a single-read sampler.
 *   data    device, 16-byte aligned; bytes a multiple of 16 (0 is a no-op).
 *   sink    device, one uint32; written only when the folded value of the
 *           data equals a fixed constant (it exists so that no load can be
 *           removed); its content is otherwise untouched.
 * Returns TES_ERR_INVALID_ARGUMENT for null or misaligned pointers or sizes,
 * TES_ERR_LAUNCH when the kernel cannot be enqueued. */
int sampler_read_probe(const void *data, uint64_t bytes, uint32_t *sink, int device,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TES_SAMPLER_H */
