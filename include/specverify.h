/*
 * specverify -- batched speculative-sampling verify step for AMD Instinct
 * MI355X (gfx950), C ABI.
 *
 * One call verifies a batch of B sequences, each with up to K drafted tokens:
 *
 *   1. temperature softmax over the vocabulary for every target position
 *      0..L_b and every draft position 0..L_b-1 of row b;
 *   2. optionally the top-p (nucleus) filter on each of those distributions;
 *   3. for j = 0..L_b-1 the acceptance test u < min(1, p'(x_j)/q'(x_j)), where
 *      the first failing j is the row's first rejection n_b (n_b = L_b if
 *      none fails);
 *   4. one more token: on a rejection, drawn from max(0, p'_n - q'_n)/Z by
 *      inverse CDF; otherwise a bonus token drawn from p'_L.
 *
 * The method is the one on the page "Speculative Decoding للمحترف: ضاعف سرعة
 * Llama 70B لـ 2.4x بدون فقد token واحد": section "المفهوم بالتقريب" (accept
 * agreed tokens, reject the first disagreeing one and resample it), section
 * "التعريف الرياضي من Leviathan et al." (the equation for the acceptance
 * probability alpha(x) = min(1, p_target(x)/p_draft(x)) and the equation for
 * the corrected distribution p'(x) = max(0, p_target(x) - p_draft(x))/Z),
 * section "كود شغّال على vLLM" (the knobs K, temperature and top_p).  The bonus
 * token is the one of the page "Faster LLM Inference via Sequential Monte
 * Carlo", section 2 (the scoring step over K+1 positions).  Per-row draft
 * lengths follow the page "HiSpec: Hierarchical Speculative Decoding for LLMs",
 * section 2 (per-sequence acceptance in a batch without padding).
 *
 * Uniforms come from Philox4x32-10 (Salmon et al., SC'11) with key = (seed low
 * word, seed high word) and counter = (row, position, 0, 0): output word 0
 * gives the acceptance uniform, word 1 the resampling uniform, each as
 * (word >> 8) * 2^-24.  Any implementation following that contract reproduces
 * the outputs bit for bit, decisions lying within rounding of a boundary
 * aside.  Precision: the softmax normalisers behind the acceptance tests are
 * float32 exponentials summed per lane and wave in float32 (relative error
 * below 1.2e-6 each, so below 2.4e-6 on p'(x)/q'(x)); the draw of step 4 is
 * float64 throughout (its own normalisers of the two rows at n, float64
 * exponentials and masses), so its token is the exact inverse-CDF token
 * unless u*Z lies within about 1e-13*Z of a boundary.
 *
 * Memory: every pointer argument is caller-owned device memory unless stated
 * otherwise.  Inputs are only read; outputs are written in full for every row.
 * The library owns a small scratch buffer per (device, stream), grown on first
 * use and kept until spec_verify_release().  Calls are asynchronous on the
 * given stream and never synchronise the host (except a first call on a
 * stream, or a call that outgrows the cached scratch, which allocates).
 *
 * Graphs: a call that does not allocate may be captured into a HIP graph:
 * each kernel of a call rewrites, before any reader needs it, all scratch
 * that later kernels of the same call read, so replays are independent.  A
 * call that would have to grow the scratch while its stream is being
 * captured returns SV_ECAPTURE and enqueues nothing (make one call of the
 * largest shape on that stream before capturing).  A buffer outgrown later
 * is kept, not freed, so graphs captured earlier stay valid;
 * spec_verify_release() frees every buffer and so invalidates every graph
 * that holds a call of this library.
 *
 * Concurrency: concurrent calls on the same stream from several host threads
 * are not supported.  Calls on different streams may run concurrently, each
 * on its stream's own scratch.  No workgroup of a call waits for another
 * workgroup to start: the row pass splits a logit row over workgroups, and
 * the one that completes the row's arrival count draws the token from the
 * records the others left, so any number of calls, and any other work on the
 * device, can share it.  A row whose record is found missing or foreign (a
 * corrupted scratch; not otherwise possible) reports out_n_accepted = -2 and
 * every token -1 (an SMC particle: bonus -2).
 *
 * Testing: with the environment variable SPECVERIFY_FAIL_LAUNCH set to a
 * non-zero value every call fails as a failed kernel launch does (SV_EHIP,
 * message through spec_verify_strerror) before touching the device.
 * SPECVERIFY_AMB_BAND (a number) replaces the relative error the row pass
 * assumes for the float32 kept-mass ratio when it classifies ids before the
 * exact ratio is known: 0 sends every row through the exact second round, a
 * wide band fills the ambiguous groups.  The result is the same either way;
 * only the path (and its time) changes.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECVERIFY_ABI_VERSION 1
#define SPECVERIFY_MAX_K 16
/* Largest vocabulary of the calls that draw a token (spec_verify,
 * spec_verify_probe, spec_smc_step, spec_hispec_verify; beyond it SV_ESHAPE).
 * Greedy verify and the draft producer take V up to 2^24. */
#define SPECVERIFY_MAX_V (1 << 21)

/* Element type of a logits tensor. */
typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Describes a device tensor of logits [B, P, V] whose V axis is contiguous.
 * Element (b, p, v) lives at data + (b*stride_b + p*stride_p + v) elements.
 * data must be aligned to the element size; strides may be anything >= 0
 * (rows need not start on 16-byte boundaries). */
typedef struct {
    const void* data;
    int32_t dtype;       /* sv_dtype */
    int32_t B, P, V;     /* P = K+1 for target logits, K for draft logits */
    int64_t stride_b;    /* elements */
    int64_t stride_p;    /* elements */
} sv_logits;

/* Status codes.  Negative values are errors. */
enum {
    SV_OK = 0,
    SV_EINVAL = -1,   /* NULL pointer, bad temperature or top_p, bad stride */
    SV_ESHAPE = -2,   /* B, K or V out of range, or the two tensors disagree */
    SV_EDTYPE = -3,   /* unknown dtype, or target and draft dtypes differ */
    SV_EHIP = -4,     /* a HIP runtime call failed; see spec_verify_strerror */
    SV_ENOMEM = -5,   /* scratch allocation failed */
    SV_EALIGN = -6,   /* a pointer is not aligned to its element size */
    SV_ECAPTURE = -7, /* the stream is being captured and the scratch would have to grow */
    SV_ETOOBIG = -8   /* spec_verify_noalloc: the call needs more than its fixed scratch */
};

/* Probe record layout (float64), per row b and position j in [0, K]:
 *   [0] target max logit          [1] target sum_v exp((l_v - max)/T)
 *   [2] draft max logit           [3] draft sum_v exp((l_v - max)/T)
 *   [4] p'(x_j), filtered target  [5] q'(x_j), filtered draft
 *   [6] kept target mass (1 when top-p is off)
 *   [7] kept draft mass  (1 when top-p is off)
 * and per row b:
 *   [0] Z, the mass the final token is drawn from
 *   [1] t = u * Z, the inverse-CDF threshold
 *   [2] u, the resampling uniform
 *   [3] n, the first-rejection index
 * Entries for positions a row does not evaluate are NaN. */
#define SV_PROBE_POS 8
#define SV_PROBE_ROW 4

/*
 * spec_verify -- the verify step (steps 1-4 above) for B rows.
 *
 * target_logits   [B, K+1, V] target logits, bf16 or fp32;
 *                 1 <= B <= 2^22, 1 <= V <= SPECVERIFY_MAX_V.
 * draft_logits    [B, K, V] draft logits, same dtype, B and V; 1 <= K <= 16.
 * draft_tokens    device int32 [B, K], contiguous; entry (b, j) is the drafted
 *                 id at position j, read only for j < L_b.
 * draft_len       device int32 [B] with L_b in [0, K], or NULL for L_b = K.
 *                 Positions >= L_b (and target positions > L_b) are never read.
 * temperature     > 0, finite; logits are divided by it before the softmax.
 * top_p           in (0, 1]; 1 switches the nucleus filter off.
 * seed            64-bit Philox key.
 * out_tokens      device int32 [B, K+1], contiguous: the n_b accepted drafted
 *                 ids, then the resampled or bonus token, then -1.
 * out_n_accepted  device int32 [B]: n_b in [0, L_b], or -1 for an invalid row
 *                 (-2: see Concurrency above; not otherwise possible).
 * stream          hipStream_t to run on (NULL = the default stream).
 *
 * Errors: arguments the host can check return SV_EINVAL / SV_ESHAPE /
 * SV_EDTYPE / SV_EALIGN and launch nothing;
 * SV_ECAPTURE as described under Graphs.  Data errors cannot be reported
 * synchronously: a row whose L_b lies outside [0, K], whose drafted id at some
 * j < L_b lies outside [0, V), or one of whose needed logit rows holds a NaN, a
 * +inf or only -inf, gets out_n_accepted = -1 and out_tokens = -1 throughout.
 * Launch failures return SV_EHIP.
 */
int spec_verify(const sv_logits* target_logits, const sv_logits* draft_logits,
                const int32_t* draft_tokens, const int32_t* draft_len,
                float temperature, float top_p, uint64_t seed,
                int32_t* out_tokens, int32_t* out_n_accepted, void* stream);

/*
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate device
 * memory (code being captured into a HIP graph, tight serving loops, hosts
 * that forbid allocation).  Same arguments, kernels and outputs as
 * spec_verify, but the scratch (statistics records, row states, candidate
 * lists, row-pass records) lives in one fixed device array of
 * SPECVERIFY_NOALLOC_SCRATCH_BYTES per device, held until the process ends,
 * so no call allocates or frees anything.  A call needing more scratch
 * returns SV_ETOOBIG and launches nothing (B = 64, K = 5, V = 128256 needs
 * about 0.4 MiB, 12.5 MiB with top-p).  Every call on a device shares that
 * device's array: calls that overlap on one device (different streams, or
 * threads) race and must not be issued; each call rewrites, before reading,
 * all the scratch it uses, so nothing needs clearing between calls.  Errors
 * otherwise as spec_verify.
 */
#define SPECVERIFY_NOALLOC_SCRATCH_BYTES (16 << 20)
int spec_verify_noalloc(const sv_logits* target_logits, const sv_logits* draft_logits,
                        const int32_t* draft_tokens, const int32_t* draft_len,
                        float temperature, float top_p, uint64_t seed,
                        int32_t* out_tokens, int32_t* out_n_accepted, void* stream);

/*
 * spec_verify_probe -- spec_verify plus the intermediate values behind each
 * decision, for testing.  probe_pos: device float64 [B, K+1, SV_PROBE_POS];
 * probe_row: device float64 [B, SV_PROBE_ROW]; layouts above.  Same errors as
 * spec_verify; the probe pointers must not be NULL.
 */
int spec_verify_probe(const sv_logits* target_logits, const sv_logits* draft_logits,
                      const int32_t* draft_tokens, const int32_t* draft_len,
                      float temperature, float top_p, uint64_t seed,
                      int32_t* out_tokens, int32_t* out_n_accepted,
                      double* probe_pos, double* probe_row, void* stream);

/*
 * spec_greedy_verify -- greedy verify: the temperature -> 0 limit of
 * spec_verify (page "Speculative Decoding للمحترف", section "المفهوم بالتقريب":
 * accept the drafted tokens the target agrees with, take the target's token at
 * the first disagreement), plus the k ids that rank after the emitted token
 * in the logits it came from (the LogitSpec page, gist.science 2507.01449,
 * section 2: candidates for the token after next; the page uses k = 60).
 *
 * target_logits   [B, K+1, V] target logits, bf16 or fp32; 1 <= K <= 16.
 * draft_tokens, draft_len: as for spec_verify (no draft logits are needed).
 * k               0 <= k <= 64.
 * out_tokens      device int32 [B, K+1]: the n accepted ids, the target's
 *                 argmax at position n (ties to the lower id), then -1.
 * out_n_accepted  device int32 [B]: n = the first j < L_b whose drafted id is
 *                 not the target's argmax (L_b if none), -1 for an invalid row.
 * out_topk        device int32 [B, k] (NULL when k = 0): the ids ranked 2..k+1
 *                 by logit at position n (descending, ties to the lower id),
 *                 -1 past V.
 *
 * Invalid rows (as for spec_verify, on the target rows 0..L_b) give n = -1
 * and -1 in every output.  Errors as spec_verify, SV_EINVAL for k outside
 * [0, 64] or out_topk NULL with k > 0.
 */
int spec_greedy_verify(const sv_logits* target_logits, const int32_t* draft_tokens,
                       const int32_t* draft_len, int32_t k, int32_t* out_tokens,
                       int32_t* out_n_accepted, int32_t* out_topk, void* stream);

/*
 * spec_hispec_verify -- the two-stage (hierarchical) verify step (page
 * "HiSpec: Hierarchical Speculative Decoding for LLMs", section 2: an
 * early-exit model's intermediate layer verifies the drafts first and rejects
 * early; the final layer verifies what passed; applying the lossless rule in
 * both stages makes the output follow the final layer exactly).
 *
 * final_logits    [B, K+2, V] final-layer logits at the positions of the
 *                 provisional sequence (positions past n1 + 1 are not read).
 * inter_logits    [B, K+1, V] intermediate-layer logits.
 * draft_logits    [B, K, V] draft-layer logits; all three the same dtype, B
 *                 and V; 1 <= K <= 15.
 * draft_tokens, draft_len, temperature, top_p, seed: as for spec_verify.
 * out_tokens      device int32 [B, K+2]: the n accepted tokens, then the
 *                 final layer's corrected or bonus token, then -1.
 * out_n_accepted  device int32 [B]: n (stage 2's accepted count), -1 for an
 *                 invalid row.
 * out_n_stage1    device int32 [B] or NULL: n1, the drafts the intermediate
 *                 layer accepted.
 *
 * Stage 1 is spec_verify(inter, draft): n1 accepted drafts and one token.
 * Stage 2 is spec_verify(final, inter) on those n1 + 1 tokens, with its
 * uniforms from Philox counter (row, position, 1, 0).  Errors as spec_verify.
 */
int spec_hispec_verify(const sv_logits* final_logits, const sv_logits* inter_logits,
                       const sv_logits* draft_logits, const int32_t* draft_tokens,
                       const int32_t* draft_len, float temperature, float top_p,
                       uint64_t seed, int32_t* out_tokens, int32_t* out_n_accepted,
                       int32_t* out_n_stage1, void* stream);

/*
 * spec_smc_step -- one reweight-and-resample step of SMC-SD over N particles
 * (page "Faster LLM Inference via Sequential Monte Carlo", section 2: every
 * particle is extended by K draft tokens and scored by the target, which also
 * yields one bonus token per particle; importance weights follow the ratio of
 * target to draft probabilities; when the effective sample size falls below a
 * threshold the particles are resampled).
 *
 * target_logits   [N, K+1, V] target logits, bf16 or fp32 (B of the
 *                 descriptor = N particles).
 * draft_logits    [N, K, V] draft logits, same dtype, N and V; 1 <= K <= 16.
 * draft_tokens    device int32 [N, K], contiguous: each particle's K drafted ids.
 * logw_in         device float64 [N]: log-weights before the step (any
 *                 common offset; -inf marks a dead particle).
 * temperature     > 0, finite; divides both models' logits (no top-p).
 * ess_fraction    resample when ESS < ess_fraction * N (0.5 is the usual
 *                 choice; <= 0 never, > 1 always resamples); not NaN.
 * seed            64-bit Philox key.  Bonus draw of particle i: word 1 of
 *                 counter (i, K, 0, 0), as the verify step's bonus; systematic
 *                 resampling offset u0: word 0 of counter (0, 0, 1, 0).
 * out_bonus       device int32 [N]: the bonus token drawn from the target at
 *                 position K by inverse CDF; -1 for an invalid particle.
 * out_logw        device float64 [N]: logw_in + sum_j (log p_j(x_j) -
 *                 log q_j(x_j)); all 0 after a resampling; -inf for an invalid
 *                 particle.  May be the same buffer as logw_in.
 * out_ancestor    device int32 [N]: the particle that slot k continues (k
 *                 itself without resampling; systematic: the first particle
 *                 whose cumulative normalised weight exceeds (k + u0)/N).
 * out_ess         device float64 [1]: (sum w)^2 / sum w^2 before resampling,
 *                 w = exp(logw - max); 0 when no particle is valid.
 * out_resampled   device int32 [1]: 1 if the step resampled.
 * stream          hipStream_t to run on (NULL = the default stream).
 *
 * A particle is invalid when a drafted id lies outside [0, V), a needed logit
 * row holds a NaN, a +inf or only -inf, or its input log-weight is NaN or
 * +inf; it never becomes an ancestor.  Host-checkable errors return
 * SV_EINVAL / SV_ESHAPE / SV_EDTYPE / SV_EALIGN and launch nothing.
 */
int spec_smc_step(const sv_logits* target_logits, const sv_logits* draft_logits,
                  const int32_t* draft_tokens, const double* logw_in,
                  float temperature, double ess_fraction, uint64_t seed,
                  int32_t* out_bonus, double* out_logw, int32_t* out_ancestor,
                  double* out_ess, int32_t* out_resampled, void* stream);

/*
 * spec_draft_produce -- the synthetic draft producer of the two-batch
 * schedule (page "MineDraft: A Framework for Batch Parallel Speculative
 * Decoding", section 2: two batches alternate, one verified while the other
 * is drafted, roles swapping every step).  The pages give no drafter; this
 * stand-in derives a batch's drafts from its target logits so that a caller
 * can run it on one stream while spec_verify runs on another:
 *
 *   draft[b, j, v] = round(float32(target[b, j, v]) + delta(b, j, v)), j < K,
 *   delta = ((h >> 5) - 1024) / 512 with h the 16-bit half (v & 1; 0 = low)
 *   of word (v & 7) >> 1 of Philox4x32-10 at counter (v >> 3, b, j, 3), key
 *   (seed low, seed high); round = round to nearest even into the logits'
 *   format (NaN stays NaN);
 *   out_tokens[b, j] = the lowest id holding the largest draft[b, j, :], or
 *   -1 when that row holds a NaN (a greedy drafter).
 *
 * target_logits  [B, P, V], bf16 or fp32; positions 0..K-1 are read.
 * K              1 <= K <= P.
 * draft_out      device buffer of the target's dtype, written at element
 *                b*out_stride_b + j*out_stride_p + v (strides in elements,
 *                >= 0); its rows must not overlap one another or the
 *                target (the library does not check this).
 * out_tokens     device int32 [B, K], contiguous.
 *
 * Errors as spec_verify: SV_EINVAL (NULL pointer, negative stride),
 * SV_ESHAPE (K outside [1, P], B or V out of range), SV_EDTYPE, SV_EALIGN,
 * SV_ENOMEM, SV_EHIP; nothing is launched on a host-checked error.  Uses the
 * stream's scratch like every other call: calls on one stream run in order.
 */
int spec_draft_produce(const sv_logits* target_logits, int32_t K, uint64_t seed,
                       void* draft_out, int64_t out_stride_b, int64_t out_stride_p,
                       int32_t* out_tokens, void* stream);

/* Human-readable text for a status code (for SV_EHIP, the last HIP error). */
const char* spec_verify_strerror(int status);

/* Frees every cached scratch buffer.  The caller must ensure no call is in
 * flight on any stream. */
void spec_verify_release(void);

/* Returns SPECVERIFY_ABI_VERSION. */
int spec_verify_abi_version(void);

/* Kernel timing for measurement.  While enabled, every launch carries a pair
 * of HIP events on its stream, attached to the kernel's dispatch.
 * spec_verify_profile_read synchronises those events and writes, for each of
 * the n kernel kinds (0 statistics pass, 1 nucleus selection, 2 row pass:
 * decision and resample, or the SMC particle pass, 3 SMC resampling, 4 the
 * synthetic draft producer), the
 * summed duration in milliseconds and the number of launches since the last
 * read; it returns the number of kinds written.  Host arrays ms[n],
 * launches[n]. */
int spec_verify_profile_enable(int enable);
int spec_verify_profile_read(double* ms, int64_t* launches, int n);

/* Measurement helper (not part of the verify step): reads every 16-byte
 * vector of the device buffer buf[0..bytes) once, with the statistics pass's
 * access pattern (workgroups of 256 threads, `unroll` in {2, 4, 8} vectors per
 * thread), so that timing it on `stream` gives the streaming-read ceiling the
 * verify kernels are measured against.  sink: device uint32[1024], written
 * only to keep the loads alive.  buf must be 16-byte aligned. */
int spec_verify_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int unroll, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
