// Internal structures shared by the host launcher and the gfx950 kernels of
// the speculative-sampling verify step.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;        // every kernel runs 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 16;
constexpr int kMaxSlots = 2 * kMaxK + 1;
constexpr int kStatsUnroll = 8;      // default 16-byte vectors in flight per lane per step
constexpr int kResTile = 8;          // consecutive ids per thread in the id-ordered scans
constexpr int kRun = 8;              // ids per thread per run of a resample item
constexpr int kRunsMax = 4;          // runs per thread per resample item, large batches
constexpr int kRunsBig = 16;         // runs per item when four-run items would not all be resident at once
constexpr int kRunIds = kThreads * kRun;  // ids per run of an item (2048)
constexpr int kRecWords = 4;         // 64-bit words per tagged statistics record
constexpr int kQKw = 24;             // word of an item's record where its per-(run, wave) sums start
// 64-bit words per row-pass item record of items of `runs` runs
constexpr int qrec_words(int runs) { return kQKw + 4 * runs * kWaves; }
constexpr int kQCnt = 21;            // word of item 0's record: the row's arrival count
constexpr int kQMass = 22;           // word of an item's record: its exact mass in a second round
constexpr int kMaxV = 1 << 21;       // largest vocabulary of the sampling entry points
constexpr int kCand = 256;           // nucleus candidates a statistics chunk lists at most
constexpr int kMaxTopK = 64;         // greedy verify: largest top-k
constexpr uint32_t kNoCover = 0xFFFFFFFFu;  // candidate header: the chunk's list covers nothing
// Exponential table of the top-p row pass for bfloat16 logits: 2^(u*c) in
// float64 for every bfloat16 u with 2^-8 <= |u| < 2^6 (biased exponents
// 119..132), entry ((bits(u) & 0x7FFF) - kTabMagLo) * 2 + sign(u).
constexpr uint32_t kTabMagLo = 119u << 7;
constexpr int kTabMags = 14 * 128;
constexpr int kTabN = 2 * kTabMags;
constexpr double kTabMaxC = 14.0;   // the table is used for c <= 14 (|u*c| < 896)

enum DType : int { DT_F32 = 0, DT_BF16 = 1 };
enum RowMode : int { MODE_SKIP = 0, MODE_RESID = 1, MODE_BONUS = 2 };
enum KernelKind : int { KK_STATS = 0, KK_TOPP = 1, KK_RESAMPLE = 2, KK_SMC = 3, KK_PRODUCE = 4, KK_COUNT = 5 };

// Statistics of one chunk of one logit row, relative to an integer offset o:
// s = sum over the chunk of 2^(l*c - o), c = log2(e)/T; m = max logit; lx =
// the logit at the row's drafted id when that id falls in the chunk, else
// -inf.  In memory a chunk's statistics are a tagged record of kRecWords
// 64-bit words (o, m, lx, s as float), each carrying the call's tag.
struct Partial {
    float o;
    float m;
    float lx;
    float s;
};

// Result of the statistics pass (and, with top-p, of the nucleus selection)
// for one logit row.  kept is the mass of the kept tokens in the same units
// as s (kept == s when the filter is off).  A token with order key k and id i
// is kept iff k > tau, or k == tau and i <= cut.
struct RvState {
    float o;
    float m;
    float lx;
    float pad0;
    double s;
    double kept;
    uint32_t tau;
    int32_t cut;
    int32_t valid;
    int32_t pad;
};

// What the resample pass needs for one batch row.
struct RowParam {
    int32_t mode;
    int32_t n;
    float oT, oD;
    double keptT, keptD;
    uint32_t tauT, tauD;
    int32_t cutT, cutD;
    double u;
};

struct Params {
    const uint8_t* tgt;
    const uint8_t* dft;
    int64_t tsb, tsp, dsb, dsp;   // strides in elements
    const int32_t* tokens;        // [B, K]
    const int32_t* dlen;          // [B] or null
    int32_t* out_tokens;          // [B, K+1]
    int32_t* out_n;               // [B]
    double* probe_pos;            // [B, K+1, 8] or null
    double* probe_row;            // [B, 4] or null
    int B, K, V, nslot;
    int nch, cv;                  // statistics pass: chunks per logit row, 16-byte vectors per chunk
    int nq;                       // resample items per batch row (runs*kRunIds ids each)
    int runs;                     // runs per resample item: 1, 2, kRunsMax or kRunsBig
    int qwords;                   // qrec_words(runs)
    uint32_t tag;                 // this call's record tag (never 0)
    float c_hi, c_lo;             // c = log2(e)/T = c_hi + c_lo, c_lo > 0 (float32 exponentials)
    double c64;                   // log2(e)/T in float64 (float64 exponentials and decisions)
    double amb_band;              // bound on the relative error of keptT/keptD from the earlier passes
    float inv_c;                  // 1/c, rounded (thresholds only)
    float top_p;
    uint32_t key0, key1;          // Philox key
    uint32_t stage;               // Philox counter word 2 of the decision (0; 1 for a second verification)
    uint64_t* prec;               // [B, nslot, nch] tagged statistics records
    RvState* rv;                  // [B, nslot]
    uint64_t* qrec;               // [B, nq, qwords] tagged row-pass item records
    double* etab;                 // [kTabN] exponential table (bfloat16 top-p calls with c <= kTabMaxC),
                                  // written by the statistics kernel, read by the row pass; else null
    // SMC-SD step (smc = 1): B particles, every one with K drafted tokens
    int smc;
    double ess_frac;              // resample when ESS < ess_frac * B
    const double* logw_in;        // [B]
    double* logw_out;             // [B] (may alias logw_in)
    int32_t* out_ancestor;        // [B]
    double* out_ess;              // [1]
    int32_t* out_resampled;       // [1]
    double* smc_cum;              // [B] scratch: cumulative normalised weights
    // greedy verify: the top-k ids after the emitted token
    int topk;
    int32_t* out_topk;            // [B, topk]
    uint64_t* chdr;               // top-p and greedy: [B, nslot, nch, kWaves, 4] tagged candidate headers (count,
                                  // key bound, key of the wave's max, lowest listed id holding it)
    uint64_t* cand;               // top-p and greedy: [B, nslot, nch, kCand] candidates (~key << 32 | id),
                                  // kCand/kWaves per wave
};

// The synthetic draft producer of the two-batch schedule (sv_produce.hip).
constexpr int kProdU = 4;  // groups of 8 ids per thread per producer workgroup
struct ProduceParams {
    const uint8_t* tgt;           // target logits [B, >= K, V]
    int64_t tsb, tsp;             // its strides (elements)
    uint8_t* out;                 // draft logits written [B, K, V], same dtype
    int64_t osb, osp;
    int32_t* tokens;              // [B, K] greedy draft tokens
    uint64_t* rec;                // [B, K, nchp, 2] scratch: tagged (key, id) per chunk
    int B, K, V, nchp;
    uint32_t k0, k1, tag;
};

// Timing events of one launch (both null when timing is off).
struct LaunchEvents {
    hipEvent_t start, stop;
};

// Launchers (defined in sv_kernels.hip).
// The statistics pass (with top-p it also lists each chunk's nucleus
// candidates), then (top-p only) the nucleus pass with the decision, then the
// row pass (decision without top-p, resample).
hipError_t launch_stats(const Params& p, int dtype, int unroll, bool topp, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_topp(const Params& p, int dtype, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_rows(const Params& p, int dtype, bool topp, hipStream_t s, const LaunchEvents& ev);
// SMC-SD step: the statistics pass, then the particle pass (log-weight
// increments and the bonus draw), then the resampling kernel.
hipError_t launch_smc_rows(const Params& p, int dtype, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_smc_resample(const Params& p, hipStream_t s, const LaunchEvents& ev);
// Greedy verify: a statistics pass of its own over the target rows (nslot =
// K + 1) that lists each wave's largest logits, then one workgroup per batch
// row.
hipError_t launch_greedy_stats(const Params& p, int dtype, int unroll, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_greedy_rows(const Params& p, int dtype, hipStream_t s, const LaunchEvents& ev);
// Two-stage verify: stage 2's draft lengths (n1 + 1) from stage 1's counts.
hipError_t launch_hispec_link(const int32_t* n1, int32_t* len2, int32_t* out_n1, int B, hipStream_t s);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int unroll, hipStream_t s);
// Synthetic draft producer: drafts and chunk records, then the tokens.
hipError_t launch_produce(const ProduceParams& p, int dtype, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_produce_tokens(const ProduceParams& p, hipStream_t s, const LaunchEvents& ev);

}  // namespace sv
