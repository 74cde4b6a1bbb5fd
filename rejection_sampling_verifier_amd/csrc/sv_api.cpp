// Host side of the specverify C ABI: argument checks, scratch management,
// kernel dispatch and optional per-kernel timing.  The operation itself is
// described in include/specverify.h.

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/specverify.h"
#include "sv_internal.h"

namespace {

using sv::Params;

struct Scratch {
    void* ptr = nullptr;       // records and per-row state; zeroed when allocated
    size_t bytes = 0;
};

static_assert(SPECVERIFY_MAX_V == sv::kMaxV, "vocabulary limit");

struct Layout {
    size_t prec, rv, qrec, chdr, cand, cum, etab, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Tagged records (statistics per chunk, masses per resample item) carry the
// call's tag; RvState is rewritten before it is read.  The top-p candidate headers and lists (present only
// when `topp`) are rewritten by the statistics pass of every top-p call.
Layout layout(int64_t B, int nslot, int nch, int nq, int qwords, bool topp, bool smc, bool tab) {
    Layout L;
    size_t off = 0;
    L.prec = off;
    off = align256(off + static_cast<size_t>(B) * nslot * nch * sv::kRecWords * sizeof(uint64_t));
    L.rv = off;
    off = align256(off + static_cast<size_t>(B) * nslot * sizeof(sv::RvState));
    L.qrec = off;
    off = align256(off + static_cast<size_t>(B) * nq * qwords * sizeof(uint64_t));
    const size_t chunks = topp ? static_cast<size_t>(B) * nslot * nch : 0;
    L.chdr = off;
    off = align256(off + chunks * sv::kWaves * 4 * sizeof(uint64_t));  // four tagged words per wave
    L.cand = off;
    off = align256(off + chunks * sv::kCand * sizeof(uint64_t));
    L.cum = off;
    off = align256(off + (smc ? static_cast<size_t>(B) * sizeof(double) : 0));
    L.etab = off;
    off = align256(off + (tab ? static_cast<size_t>(sv::kTabN) * sizeof(double) : 0));
    L.total = off;
    return L;
}

// Record tags: unique per call within the process, never 0.
std::atomic<uint32_t> g_tag{0};
uint32_t next_tag() {
    uint32_t t;
    do {
        t = g_tag.fetch_add(1u) + 1u;
    } while (t == 0u);
    return t;
}

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;
thread_local std::string g_hip_msg;

struct EvPair {
    hipEvent_t a, b;
    int kind;
};
bool g_prof = false;
std::vector<EvPair> g_events;

int hip_fail(hipError_t e, const char* what) {
    g_hip_msg = std::string(what) + ": " + hipGetErrorString(e);
    return SV_EHIP;
}

int env_int(const char* name, int dflt) {
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    return std::atoi(s);
}

double env_double(const char* name, double dflt) {
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    return std::atof(s);
}

bool misaligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Compute units of the current device (cached per device).
int device_cus() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
    return n;
}

int check_logits(const sv_logits* t) {
    if (!t || !t->data) return SV_EINVAL;
    if (t->dtype != SV_F32 && t->dtype != SV_BF16) return SV_EDTYPE;
    if (t->stride_b < 0 || t->stride_p < 0) return SV_EINVAL;
    if (misaligned(t->data, t->dtype == SV_BF16 ? 2 : 4)) return SV_EALIGN;
    return SV_OK;
}

// Test-only fault injection: with SPECVERIFY_FAIL_LAUNCH set to a non-zero
// value every call fails where it would first touch the device, as a failed
// launch does (SV_EHIP and its message), so that the error path can be
// tested without a GPU.
bool fail_launch_forced() { return env_int("SPECVERIFY_FAIL_LAUNCH", 0) != 0; }

// Scratch of spec_verify_noalloc: one fixed array per device, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocBytes = static_cast<size_t>(SPECVERIFY_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];
std::mutex g_noalloc_mu;
std::map<int, void*> g_noalloc_ptr;

int noalloc_scratch(void** out) {
    if (fail_launch_forced()) return hip_fail(hipErrorLaunchFailure, "kernel launch (forced by SPECVERIFY_FAIL_LAUNCH)");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    auto it = g_noalloc_ptr.find(dev);
    if (it == g_noalloc_ptr.end()) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        it = g_noalloc_ptr.emplace(dev, ptr).first;
    }
    *out = it->second;
    return SV_OK;
}

// Buffers replaced by larger ones.  A HIP graph captured from an earlier
// call may still use them, so they are freed only by spec_verify_release.
std::vector<void*> g_retired;

// Returns the scratch for (device, stream), growing it (zeroed) when needed.
// Growing allocates and synchronises the stream, which a stream being
// captured into a graph cannot do: then SV_ECAPTURE, and nothing changes.
int get_scratch(hipStream_t stream, size_t bytes, void** data) {
    if (fail_launch_forced()) return hip_fail(hipErrorLaunchFailure, "kernel launch (forced by SPECVERIFY_FAIL_LAUNCH)");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_mu);
    Scratch& s = g_scratch[{dev, stream}];
    if (s.bytes >= bytes) {
        *data = s.ptr;
        return SV_OK;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone) return SV_ECAPTURE;
    if (s.ptr) {
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    }
    void* p = nullptr;
    const size_t want = bytes + bytes / 4;
    e = hipMalloc(&p, want);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return SV_ENOMEM;
    }
    e = hipMemsetAsync(p, 0, want, stream);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return hip_fail(e, "hipMemsetAsync");
    }
    if (s.ptr) g_retired.push_back(s.ptr);
    s.ptr = p;
    s.bytes = want;
    *data = s.ptr;
    return SV_OK;
}

template <typename F>
int timed_launch(int kind, hipStream_t stream, F&& launch) {
    EvPair ev{nullptr, nullptr, kind};
    if (g_prof) {
        if (hipEventCreate(&ev.a) != hipSuccess || hipEventCreate(&ev.b) != hipSuccess)
            return hip_fail(hipGetLastError(), "hipEventCreate");
    }
    if (fail_launch_forced()) return hip_fail(hipErrorLaunchFailure, "kernel launch (forced by SPECVERIFY_FAIL_LAUNCH)");
    const hipError_t e = launch(sv::LaunchEvents{ev.a, ev.b});
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    if (g_prof) {
        std::lock_guard<std::mutex> lk(g_mu);
        g_events.push_back(ev);
    }
    return SV_OK;
}

// What every entry point shares: argument checks, chunking and the kernel
// parameters (plan), then the scratch pointers (bind).  `smc`: an SMC-SD step
// (no draft lengths, no top-p, the resampling kernel's scratch).
struct Setup {
    Params p;
    int dtype = 0;
    int unroll = 0;
    bool topp = false;
    hipStream_t stream = nullptr;
    Layout lay;
    bool tab = false;
};

enum Mode { MODE_VERIFY = 0, MODE_SMC = 1, MODE_GREEDY = 2 };

int plan(const sv_logits* tl, const sv_logits* dl, const int32_t* draft_tokens, const int32_t* draft_len,
         float temperature, float top_p, uint64_t seed, int mode, void* stream_v, Setup& S) {
    const bool smc = mode == MODE_SMC, greedy = mode == MODE_GREEDY;
    int rc = check_logits(tl);
    if (rc) return rc;
    if (!greedy) {
        rc = check_logits(dl);
        if (rc) return rc;
    }
    if (!draft_tokens) return SV_EINVAL;
    if (misaligned(draft_tokens, 4) || (draft_len && misaligned(draft_len, 4))) return SV_EALIGN;
    if (!greedy && tl->dtype != dl->dtype) return SV_EDTYPE;
    const int B = tl->B, V = tl->V, K = tl->P - 1;
    if (B <= 0 || V <= 0 || K < 1 || K > SPECVERIFY_MAX_K) return SV_ESHAPE;
    if (!greedy && (dl->B != B || dl->V != V || dl->P != K)) return SV_ESHAPE;
    if (B > (1 << 22) || V > (greedy ? (1 << 24) : SPECVERIFY_MAX_V)) return SV_ESHAPE;
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return SV_EINVAL;
    if (!(top_p > 0.f && top_p <= 1.f)) return SV_EINVAL;
    const double c = 1.4426950408889634074 / static_cast<double>(temperature);  // log2(e)/T
    if (!(c < static_cast<double>(FLT_MAX))) return SV_EINVAL;

    const int dtype = tl->dtype == SV_BF16 ? sv::DT_BF16 : sv::DT_F32;
    const int E = dtype == sv::DT_BF16 ? 2 : 4;
    // greedy verify reads the target rows only
    const int nslot = greedy ? K + 1 : 2 * K + 1;
    // statistics pass: chunks of at most `cv` 16-byte vectors per workgroup
    const int64_t nvec_max = (static_cast<int64_t>(V) * E + 15) / 16 + 1;
    int unroll = env_int("SPECVERIFY_STATS_UNROLL", sv::kStatsUnroll);
    if (unroll != 4) unroll = 8;
    // a statistics workgroup reads one chunk of kThreads*unroll vectors; only
    // a row's last chunk is partial
    const int cv = sv::kThreads * unroll;
    const int64_t nch64 = (nvec_max + cv - 1) / cv;
    const int nch = static_cast<int>(nch64);
    // row pass: items of runs*kRunIds ids.  Four-run items by default; one-run
    // items when the batch would otherwise give fewer than two workgroups per
    // CU; sixteen-run items when four-run items would not all be resident at
    // once (four workgroups per CU), so that every row pays the pass's latency
    // chain once instead of once per round of workgroups
    int runs = sv::kRunsMax;
    if (!greedy) {
        const int cus = device_cus();
        auto items = [&](int ru) { return static_cast<int64_t>(B) * ((V + ru * sv::kRunIds - 1) / (ru * sv::kRunIds)); };
        if (items(runs) < 2ll * cus) runs = 1;
        else if (items(runs) > 4ll * cus && items(sv::kRunsBig) < items(runs)) runs = sv::kRunsBig;
        const int forced = env_int("SPECVERIFY_ROW_RUNS", 0);
        if (forced == 1 || forced == 2 || forced == sv::kRunsMax || forced == sv::kRunsBig) runs = forced;
    }
    const int nq = greedy ? 0 : (V + runs * sv::kRunIds - 1) / (runs * sv::kRunIds);
    const int qwords = sv::qrec_words(runs);
    const int64_t per_row = static_cast<int64_t>(nslot) * nch + nq;
    if (static_cast<int64_t>(B) * per_row >= (1ll << 31)) return SV_ESHAPE;
    // the statistics kernel clears the row pass's records, a few words each
    if (static_cast<int64_t>(qwords) * nq > static_cast<int64_t>(sv::kThreads) * nslot * nch) return SV_ESHAPE;

    // greedy verify takes its argmaxes and top-k from the candidate lists
    const bool topp = top_p < 1.f || greedy;
    // the top-p row pass's exponential table (bfloat16 rows; for larger c its
    // entries 2^(u*c) would leave the float64 range)
    S.tab = dtype == sv::DT_BF16 && !greedy && !smc && top_p < 1.f && c <= sv::kTabMaxC;
    S.lay = layout(B, nslot, nch, nq, qwords, topp, smc, S.tab);

    Params& p = S.p;
    std::memset(&p, 0, sizeof(p));
    p.tgt = static_cast<const uint8_t*>(tl->data);
    p.tsb = tl->stride_b;
    p.tsp = tl->stride_p;
    if (!greedy) {
        p.dft = static_cast<const uint8_t*>(dl->data);
        p.dsb = dl->stride_b;
        p.dsp = dl->stride_p;
    }
    p.tokens = draft_tokens;
    p.dlen = draft_len;
    p.B = B;
    p.K = K;
    p.V = V;
    p.nslot = nslot;
    p.nch = nch;
    p.cv = cv;
    p.nq = nq;
    p.runs = runs;
    p.qwords = qwords;
    p.tag = next_tag();
    // c = c_hi + c_lo with c_hi <= c rounded toward zero, so c_lo > 0.
    float c_hi = static_cast<float>(c);
    if (static_cast<double>(c_hi) > c) c_hi = std::nextafter(c_hi, 0.f);
    float c_lo = static_cast<float>(c - static_cast<double>(c_hi));
    if (!(c_lo >= FLT_MIN)) c_lo = FLT_MIN;
    p.c_hi = c_hi;
    p.c_lo = c_lo;
    p.c64 = c;
    // relative error bound of keptT/keptD as the statistics (and nucleus)
    // passes compute them: float32 exponentials and float32 lane and wave
    // sums, below 1.2e-6 per normaliser (below 2e-6 per kept mass)
    // SPECVERIFY_AMB_BAND replaces it (tests: 0 sends every row to the exact
    // second round, a wide band fills the items' ambiguous groups)
    p.amb_band = env_double("SPECVERIFY_AMB_BAND", top_p < 1.f ? 4e-6 : 2.5e-6);
    p.inv_c = static_cast<float>(1.0 / c);
    p.top_p = top_p;
    p.key0 = static_cast<uint32_t>(seed & 0xFFFFFFFFull);
    p.key1 = static_cast<uint32_t>(seed >> 32);
    p.smc = smc ? 1 : 0;
    S.dtype = dtype;
    S.unroll = unroll;
    S.topp = topp;
    S.stream = static_cast<hipStream_t>(stream_v);
    return SV_OK;
}

void bind(Setup& S, uint8_t* base) {
    Params& p = S.p;
    const Layout& lay = S.lay;
    p.prec = reinterpret_cast<uint64_t*>(base + lay.prec);
    p.rv = reinterpret_cast<sv::RvState*>(base + lay.rv);
    p.qrec = reinterpret_cast<uint64_t*>(base + lay.qrec);
    p.chdr = S.topp ? reinterpret_cast<uint64_t*>(base + lay.chdr) : nullptr;
    p.cand = S.topp ? reinterpret_cast<uint64_t*>(base + lay.cand) : nullptr;
    p.smc_cum = p.smc ? reinterpret_cast<double*>(base + lay.cum) : nullptr;
    p.etab = S.tab ? reinterpret_cast<double*>(base + lay.etab) : nullptr;
}

// plan + scratch + bind for a single pass.
int prepare(const sv_logits* tl, const sv_logits* dl, const int32_t* draft_tokens, const int32_t* draft_len,
            float temperature, float top_p, uint64_t seed, int mode, void* stream_v, Setup& S) {
    int rc = plan(tl, dl, draft_tokens, draft_len, temperature, top_p, seed, mode, stream_v, S);
    if (rc) return rc;
    void* scratch = nullptr;
    rc = get_scratch(S.stream, S.lay.total, &scratch);
    if (rc) return rc;
    bind(S, static_cast<uint8_t*>(scratch));
    return SV_OK;
}

// The verify step's kernels for one planned and bound pass.
int launch_verify(Setup& S) {
    Params& p = S.p;
    const hipStream_t stream = S.stream;
    int rc = timed_launch(sv::KK_STATS, stream, [&](const sv::LaunchEvents& ev) {
        return sv::launch_stats(p, S.dtype, S.unroll, S.topp, stream, ev);
    });
    if (rc) return rc;
    if (S.topp) {
        rc = timed_launch(sv::KK_TOPP, stream,
                          [&](const sv::LaunchEvents& ev) { return sv::launch_topp(p, S.dtype, stream, ev); });
        if (rc) return rc;
    }
    return timed_launch(sv::KK_RESAMPLE, stream,
                        [&](const sv::LaunchEvents& ev) { return sv::launch_rows(p, S.dtype, S.topp, stream, ev); });
}

int verify_impl(const sv_logits* tl, const sv_logits* dl, const int32_t* draft_tokens, const int32_t* draft_len,
                float temperature, float top_p, uint64_t seed, int32_t* out_tokens, int32_t* out_n,
                double* probe_pos, double* probe_row, void* stream_v) {
    if (!out_tokens || !out_n) return SV_EINVAL;
    if (misaligned(out_tokens, 4) || misaligned(out_n, 4)) return SV_EALIGN;
    Setup S;
    int rc = prepare(tl, dl, draft_tokens, draft_len, temperature, top_p, seed, MODE_VERIFY, stream_v, S);
    if (rc) return rc;
    S.p.out_tokens = out_tokens;
    S.p.out_n = out_n;
    S.p.probe_pos = probe_pos;
    S.p.probe_row = probe_row;
    return launch_verify(S);
}

// spec_verify on the fixed per-device scratch: the same kernels, no
// allocation; calls needing more than the array holds are refused.
int verify_noalloc_impl(const sv_logits* tl, const sv_logits* dl, const int32_t* draft_tokens,
                        const int32_t* draft_len, float temperature, float top_p, uint64_t seed, int32_t* out_tokens,
                        int32_t* out_n, void* stream_v) {
    if (!out_tokens || !out_n) return SV_EINVAL;
    if (misaligned(out_tokens, 4) || misaligned(out_n, 4)) return SV_EALIGN;
    Setup S;
    int rc = plan(tl, dl, draft_tokens, draft_len, temperature, top_p, seed, MODE_VERIFY, stream_v, S);
    if (rc) return rc;
    if (S.lay.total > kNoAllocBytes) return SV_ETOOBIG;
    void* base = nullptr;
    rc = noalloc_scratch(&base);
    if (rc) return rc;
    bind(S, static_cast<uint8_t*>(base));
    S.p.out_tokens = out_tokens;
    S.p.out_n = out_n;
    return launch_verify(S);
}

// Two-stage verify: stage 1 verifies the drafts against the intermediate
// layer, stage 2 the n1 + 1 tokens it emitted against the final layer (the
// intermediate layer as their proposal, Philox stream 1).  One scratch
// allocation holds both passes' regions and stage 1's outputs.
int hispec_impl(const sv_logits* fl, const sv_logits* il, const sv_logits* dl, const int32_t* draft_tokens,
                const int32_t* draft_len, float temperature, float top_p, uint64_t seed, int32_t* out_tokens,
                int32_t* out_n, int32_t* out_n_stage1, void* stream_v) {
    if (!out_tokens || !out_n) return SV_EINVAL;
    if (misaligned(out_tokens, 4) || misaligned(out_n, 4) || (out_n_stage1 && misaligned(out_n_stage1, 4)))
        return SV_EALIGN;
    if (!fl || !il) return SV_EINVAL;
    if (fl->B != il->B || fl->V != il->V || fl->P != il->P + 1) return SV_ESHAPE;
    Setup S1, S2;
    int rc = plan(il, dl, draft_tokens, draft_len, temperature, top_p, seed, MODE_VERIFY, stream_v, S1);
    if (rc) return rc;
    // stage 2's drafts are device scratch bound below; the caller's ids stand
    // in for the host checks
    rc = plan(fl, il, draft_tokens, nullptr, temperature, top_p, seed, MODE_VERIFY, stream_v, S2);
    if (rc) return rc;
    const int B = S1.p.B, K1 = S1.p.K + 1;
    const size_t tok_bytes = align256(static_cast<size_t>(B) * K1 * sizeof(int32_t));
    const size_t vec_bytes = align256(static_cast<size_t>(B) * sizeof(int32_t));
    const size_t total = S1.lay.total + S2.lay.total + tok_bytes + 2 * vec_bytes;
    void* scratch = nullptr;
    rc = get_scratch(S1.stream, total, &scratch);
    if (rc) return rc;
    uint8_t* base = static_cast<uint8_t*>(scratch);
    bind(S1, base);
    bind(S2, base + S1.lay.total);
    uint8_t* extra = base + S1.lay.total + S2.lay.total;
    int32_t* tok1 = reinterpret_cast<int32_t*>(extra);
    int32_t* n1 = reinterpret_cast<int32_t*>(extra + tok_bytes);
    int32_t* len2 = reinterpret_cast<int32_t*>(extra + tok_bytes + vec_bytes);
    S1.p.out_tokens = tok1;
    S1.p.out_n = n1;
    S2.p.tokens = tok1;
    S2.p.dlen = len2;
    S2.p.stage = 1;
    S2.p.out_tokens = out_tokens;
    S2.p.out_n = out_n;
    rc = launch_verify(S1);
    if (rc) return rc;
    const hipError_t e = sv::launch_hispec_link(n1, len2, out_n_stage1, B, S1.stream);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return launch_verify(S2);
}

// Greedy verify: the statistics pass over the target rows with candidate
// lists (at T = 1, which only scales the list bins), then one workgroup per
// batch row for the argmaxes, the decision and the top-k.
int greedy_impl(const sv_logits* tl, const int32_t* draft_tokens, const int32_t* draft_len, int32_t k,
                int32_t* out_tokens, int32_t* out_n, int32_t* out_topk, void* stream_v) {
    if (!out_tokens || !out_n || (k > 0 && !out_topk)) return SV_EINVAL;
    if (k < 0 || k > sv::kMaxTopK) return SV_EINVAL;
    if (misaligned(out_tokens, 4) || misaligned(out_n, 4) || (out_topk && misaligned(out_topk, 4))) return SV_EALIGN;
    Setup S;
    int rc = prepare(tl, nullptr, draft_tokens, draft_len, 1.f, 1.f, 0, MODE_GREEDY, stream_v, S);
    if (rc) return rc;
    Params& p = S.p;
    p.out_tokens = out_tokens;
    p.out_n = out_n;
    p.topk = k;
    p.out_topk = out_topk;
    const hipStream_t stream = S.stream;
    rc = timed_launch(sv::KK_STATS, stream, [&](const sv::LaunchEvents& ev) {
        return sv::launch_greedy_stats(p, S.dtype, S.unroll, stream, ev);
    });
    if (rc) return rc;
    return timed_launch(sv::KK_RESAMPLE, stream,
                        [&](const sv::LaunchEvents& ev) { return sv::launch_greedy_rows(p, S.dtype, stream, ev); });
}

int smc_impl(const sv_logits* tl, const sv_logits* dl, const int32_t* draft_tokens, const double* logw_in,
             float temperature, double ess_fraction, uint64_t seed, int32_t* out_bonus, double* out_logw,
             int32_t* out_ancestor, double* out_ess, int32_t* out_resampled, void* stream_v) {
    if (!logw_in || !out_bonus || !out_logw || !out_ancestor || !out_ess || !out_resampled) return SV_EINVAL;
    if (misaligned(logw_in, 8) || misaligned(out_logw, 8) || misaligned(out_ess, 8) || misaligned(out_bonus, 4) ||
        misaligned(out_ancestor, 4) || misaligned(out_resampled, 4))
        return SV_EALIGN;
    if (std::isnan(ess_fraction)) return SV_EINVAL;
    Setup S;
    int rc = prepare(tl, dl, draft_tokens, nullptr, temperature, 1.f, seed, MODE_SMC, stream_v, S);
    if (rc) return rc;
    Params& p = S.p;
    p.out_tokens = out_bonus;
    p.ess_frac = ess_fraction;
    p.logw_in = logw_in;
    p.logw_out = out_logw;
    p.out_ancestor = out_ancestor;
    p.out_ess = out_ess;
    p.out_resampled = out_resampled;
    const hipStream_t stream = S.stream;
    rc = timed_launch(sv::KK_STATS, stream, [&](const sv::LaunchEvents& ev) {
        return sv::launch_stats(p, S.dtype, S.unroll, false, stream, ev);
    });
    if (rc) return rc;
    rc = timed_launch(sv::KK_RESAMPLE, stream,
                      [&](const sv::LaunchEvents& ev) { return sv::launch_smc_rows(p, S.dtype, stream, ev); });
    if (rc) return rc;
    return timed_launch(sv::KK_SMC, stream,
                        [&](const sv::LaunchEvents& ev) { return sv::launch_smc_resample(p, stream, ev); });
}

// Synthetic draft producer of the two-batch schedule: drafts and chunk
// records, then the tokens.  Its chunk records use the (device, stream)
// scratch like every other call on that stream.
int produce_impl(const sv_logits* tl, int32_t K, uint64_t seed, void* out, int64_t osb, int64_t osp,
                 int32_t* out_tokens, void* stream_v) {
    int rc = check_logits(tl);
    if (rc) return rc;
    if (!out || !out_tokens) return SV_EINVAL;
    const int E = tl->dtype == SV_BF16 ? 2 : 4;
    if (misaligned(out, E) || misaligned(out_tokens, 4)) return SV_EALIGN;
    if (osb < 0 || osp < 0) return SV_EINVAL;
    const int B = tl->B, V = tl->V;
    if (B <= 0 || V <= 0 || K < 1 || K > tl->P || B > (1 << 22) || V > (1 << 24)) return SV_ESHAPE;
    const int64_t groups = (static_cast<int64_t>(V) + 7) / 8;
    const int64_t per = static_cast<int64_t>(sv::kThreads) * sv::kProdU;
    const int nchp = static_cast<int>((groups + per - 1) / per);
    if (static_cast<int64_t>(B) * K * nchp >= (1ll << 31)) return SV_ESHAPE;
    const hipStream_t stream = static_cast<hipStream_t>(stream_v);
    void* base = nullptr;
    rc = get_scratch(stream, static_cast<size_t>(B) * K * nchp * 2 * sizeof(uint64_t), &base);
    if (rc) return rc;
    sv::ProduceParams p;
    std::memset(&p, 0, sizeof(p));
    p.tgt = static_cast<const uint8_t*>(tl->data);
    p.tsb = tl->stride_b;
    p.tsp = tl->stride_p;
    p.out = static_cast<uint8_t*>(out);
    p.osb = osb;
    p.osp = osp;
    p.tokens = out_tokens;
    p.rec = static_cast<uint64_t*>(base);
    p.B = B;
    p.K = K;
    p.V = V;
    p.nchp = nchp;
    p.k0 = static_cast<uint32_t>(seed);
    p.k1 = static_cast<uint32_t>(seed >> 32);
    p.tag = next_tag();
    const int dtype = tl->dtype == SV_BF16 ? sv::DT_BF16 : sv::DT_F32;
    rc = timed_launch(sv::KK_PRODUCE, stream,
                      [&](const sv::LaunchEvents& ev) { return sv::launch_produce(p, dtype, stream, ev); });
    if (rc) return rc;
    return timed_launch(sv::KK_PRODUCE, stream,
                        [&](const sv::LaunchEvents& ev) { return sv::launch_produce_tokens(p, stream, ev); });
}

}  // namespace

extern "C" {

int spec_verify(const sv_logits* target_logits, const sv_logits* draft_logits, const int32_t* draft_tokens,
                const int32_t* draft_len, float temperature, float top_p, uint64_t seed, int32_t* out_tokens,
                int32_t* out_n_accepted, void* stream) {
    return verify_impl(target_logits, draft_logits, draft_tokens, draft_len, temperature, top_p, seed, out_tokens,
                       out_n_accepted, nullptr, nullptr, stream);
}

int spec_verify_noalloc(const sv_logits* target_logits, const sv_logits* draft_logits, const int32_t* draft_tokens,
                        const int32_t* draft_len, float temperature, float top_p, uint64_t seed, int32_t* out_tokens,
                        int32_t* out_n_accepted, void* stream) {
    return verify_noalloc_impl(target_logits, draft_logits, draft_tokens, draft_len, temperature, top_p, seed,
                               out_tokens, out_n_accepted, stream);
}

int spec_verify_probe(const sv_logits* target_logits, const sv_logits* draft_logits, const int32_t* draft_tokens,
                      const int32_t* draft_len, float temperature, float top_p, uint64_t seed,
                      int32_t* out_tokens, int32_t* out_n_accepted, double* probe_pos, double* probe_row,
                      void* stream) {
    if (!probe_pos || !probe_row) return SV_EINVAL;
    if (misaligned(probe_pos, 8) || misaligned(probe_row, 8)) return SV_EALIGN;
    return verify_impl(target_logits, draft_logits, draft_tokens, draft_len, temperature, top_p, seed, out_tokens,
                       out_n_accepted, probe_pos, probe_row, stream);
}

int spec_greedy_verify(const sv_logits* target_logits, const int32_t* draft_tokens, const int32_t* draft_len,
                       int32_t k, int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_topk, void* stream) {
    return greedy_impl(target_logits, draft_tokens, draft_len, k, out_tokens, out_n_accepted, out_topk, stream);
}

int spec_hispec_verify(const sv_logits* final_logits, const sv_logits* inter_logits, const sv_logits* draft_logits,
                       const int32_t* draft_tokens, const int32_t* draft_len, float temperature, float top_p,
                       uint64_t seed, int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_n_stage1,
                       void* stream) {
    return hispec_impl(final_logits, inter_logits, draft_logits, draft_tokens, draft_len, temperature, top_p, seed,
                       out_tokens, out_n_accepted, out_n_stage1, stream);
}

int spec_smc_step(const sv_logits* target_logits, const sv_logits* draft_logits, const int32_t* draft_tokens,
                  const double* logw_in, float temperature, double ess_fraction, uint64_t seed, int32_t* out_bonus,
                  double* out_logw, int32_t* out_ancestor, double* out_ess, int32_t* out_resampled, void* stream) {
    return smc_impl(target_logits, draft_logits, draft_tokens, logw_in, temperature, ess_fraction, seed, out_bonus,
                    out_logw, out_ancestor, out_ess, out_resampled, stream);
}

int spec_draft_produce(const sv_logits* target_logits, int32_t K, uint64_t seed, void* draft_out,
                       int64_t out_stride_b, int64_t out_stride_p, int32_t* out_tokens, void* stream) {
    return produce_impl(target_logits, K, seed, draft_out, out_stride_b, out_stride_p, out_tokens, stream);
}

const char* spec_verify_strerror(int status) {
    switch (status) {
        case SV_OK: return "success";
        case SV_EINVAL: return "invalid argument (NULL pointer, temperature, top_p or stride)";
        case SV_ESHAPE: return "invalid shape (B, K, V out of range or target/draft mismatch)";
        case SV_EDTYPE: return "invalid or mismatched dtype";
        case SV_EHIP: return g_hip_msg.empty() ? "HIP runtime error" : g_hip_msg.c_str();
        case SV_ENOMEM: return "scratch allocation failed";
        case SV_EALIGN: return "pointer not aligned to its element size";
        case SV_ECAPTURE: return "the stream is being captured and the call would have to grow its scratch";
        case SV_ETOOBIG: return "the call needs more scratch than spec_verify_noalloc's fixed array holds";
        default: return "unknown status";
    }
}

void spec_verify_release(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& kv : g_scratch) {
        if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    }
    g_scratch.clear();
    for (void* p : g_retired) (void)hipFree(p);
    g_retired.clear();
}

int spec_verify_abi_version(void) { return SPECVERIFY_ABI_VERSION; }

int spec_verify_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int unroll, void* stream) {
    if (!buf || !sink || bytes < 16) return SV_EINVAL;
    if (misaligned(buf, 16) || misaligned(sink, 4)) return SV_EALIGN;
    if (unroll != 2 && unroll != 4 && unroll != 8) return SV_EINVAL;
    const hipError_t e = sv::launch_stream_read(buf, bytes, sink, unroll, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SV_OK : hip_fail(e, "stream read launch");
}

int spec_verify_profile_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_prof = enable != 0;
    return SV_OK;
}

int spec_verify_profile_read(double* ms, int64_t* launches, int n) {
    if (n < 0 || (n > 0 && (!ms || !launches))) return SV_EINVAL;
    std::vector<EvPair> evs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        evs.swap(g_events);
    }
    const int kinds = n < sv::KK_COUNT ? n : sv::KK_COUNT;
    for (int k = 0; k < kinds; ++k) {
        ms[k] = 0.0;
        launches[k] = 0;
    }
    int rc = SV_OK;
    for (const EvPair& e : evs) {
        float t = 0.f;
        hipError_t err = hipEventSynchronize(e.b);
        if (err == hipSuccess) err = hipEventElapsedTime(&t, e.a, e.b);
        if (err != hipSuccess) rc = hip_fail(err, "hipEventElapsedTime");
        if (e.kind < kinds) {
            ms[e.kind] += t;
            launches[e.kind] += 1;
        }
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    return rc == SV_OK ? kinds : rc;
}

}  // extern "C"
