// gfx950 kernels of the synthetic draft producer of the two-batch schedule
// (page "MineDraft: A Framework for Batch Parallel Speculative Decoding",
// section 2, the alternation between batches: while the target verifies one
// batch, the drafter drafts the other, and the roles swap every step).  The
// pages give no drafter; this stand-in writes, for every batch row b and
// draft position j < K,
//
//   draft[b, j, v] = round(float32(target[b, j, v]) + delta(b, j, v)),
//   delta = ((h >> 5) - 1024) / 512, h = 16-bit half (v & 1) of word
//           (v & 7) >> 1 of Philox4x32-10 at counter (v >> 3, b, j, 3),
//
// rounded to the logits' format (round to nearest even for bf16), and the
// greedy token of each draft row: the lowest id of its largest logit, -1 if
// the row holds a NaN.
//
//   k_produce         one workgroup per (b, j, chunk of 8192 ids): one
//                     Philox call per 8 ids, 16-byte loads and stores when
//                     both rows are aligned; a tagged (key, id) record of
//                     the chunk's largest draft logit.
//   k_produce_tokens  one wave per (b, j): the largest of the row's chunk
//                     records, read by the lanes in parallel.

#include <hip/hip_ext.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kProdIds = 8;  // ids per Philox call
constexpr uint32_t kProdNaN = 0xFFFFFFFFu;  // record key of a chunk holding a NaN

__device__ __forceinline__ uint32_t prod_word(const uint4& r, int q) {
    return q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
}

// float32 -> bf16 bits, round to nearest even, NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float s) {
    const uint32_t u = __float_as_uint(s);
    return __builtin_isnan(s) ? 0x7FC0u : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_produce(ProduceParams P) {
    constexpr int E = Fmt<DT>::E;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int item = blockIdx.x;
    const int rj = item / P.nchp;
    const int chunk = item - rj * P.nchp;
    const int b = rj / P.K, j = rj - b * P.K;
    const uint8_t* src = P.tgt + (static_cast<int64_t>(b) * P.tsb + static_cast<int64_t>(j) * P.tsp) * E;
    uint8_t* dst = P.out + (static_cast<int64_t>(b) * P.osb + static_cast<int64_t>(j) * P.osp) * E;
    const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    uint64_t best = 0ull;  // (order key << 32) | (~id): the largest logit, then the lowest id
    bool nan = false;
#pragma unroll
    for (int u = 0; u < kProdU; ++u) {
        const int64_t g = (static_cast<int64_t>(chunk) * kProdU + u) * kThreads + tid;
        const int64_t id0 = g * kProdIds;
        if (id0 >= P.V) continue;
        const bool full = vec && id0 + kProdIds <= P.V;
        float t[kProdIds];
        if (full) {
            if (DT == DT_BF16) {
                const uint4 v = gload16(reinterpret_cast<const uint4*>(src) + g);
#pragma unroll
                for (int i = 0; i < kProdIds; ++i) {
                    const uint32_t w = prod_word(v, i >> 1);
                    t[i] = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
                }
            } else {
                const uint4 v0 = gload16(reinterpret_cast<const uint4*>(src) + 2 * g);
                const uint4 v1 = gload16(reinterpret_cast<const uint4*>(src) + 2 * g + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    t[i] = __uint_as_float(prod_word(v0, i));
                    t[4 + i] = __uint_as_float(prod_word(v1, i));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kProdIds; ++i) t[i] = id0 + i < P.V ? load_elem<DT>(src, id0 + i) : 0.f;
        }
        const uint4 r = philox4x32_10(make_uint4(static_cast<uint32_t>(g), static_cast<uint32_t>(b),
                                                 static_cast<uint32_t>(j), 3u),
                                      P.k0, P.k1);
        uint32_t o[kProdIds];
#pragma unroll
        for (int i = 0; i < kProdIds; ++i) {
            const uint32_t w = prod_word(r, i >> 1);
            const uint32_t h = (i & 1) ? (w >> 16) : (w & 0xFFFFu);
            const float d = static_cast<float>(static_cast<int>(h >> 5) - 1024) * (1.f / 512.f);
            const float s = t[i] + d;
            float val;
            if (DT == DT_BF16) {
                o[i] = bf16_rne(s);
                val = __uint_as_float(o[i] << 16);
            } else {
                o[i] = __float_as_uint(s);
                val = s;
            }
            if (id0 + i < P.V) {
                if (__builtin_isnan(val)) nan = true;
                const uint64_t pk = (static_cast<uint64_t>(order_key(val)) << 32) |
                                    static_cast<uint32_t>(~static_cast<uint32_t>(id0 + i));
                best = pk > best ? pk : best;
            }
        }
        if (full) {
            if (DT == DT_BF16) {
                reinterpret_cast<uint4*>(dst)[g] =
                    make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16));
            } else {
                reinterpret_cast<uint4*>(dst)[2 * g] = make_uint4(o[0], o[1], o[2], o[3]);
                reinterpret_cast<uint4*>(dst)[2 * g + 1] = make_uint4(o[4], o[5], o[6], o[7]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kProdIds; ++i) {
                if (id0 + i < P.V) {
                    if (DT == DT_BF16) reinterpret_cast<uint16_t*>(dst)[id0 + i] = static_cast<uint16_t>(o[i]);
                    else reinterpret_cast<uint32_t*>(dst)[id0 + i] = o[i];
                }
            }
        }
    }
    // workgroup max of the packed (key, ~id)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(best), off, 64);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(best >> 32), off, 64);
        const uint64_t ob = (static_cast<uint64_t>(hi) << 32) | lo;
        best = ob > best ? ob : best;
    }
    const bool nanw = __ballot(nan) != 0ull;
    __shared__ uint64_t s_best[kWaves];
    __shared__ int s_nan[kWaves];
    if (lane == 0) {
        s_best[wv] = best;
        s_nan[wv] = nanw ? 1 : 0;
    }
    __syncthreads();
    if (tid < 2) {
        uint64_t bb = s_best[0];
        int nn = s_nan[0];
        for (int w = 1; w < kWaves; ++w) {
            bb = s_best[w] > bb ? s_best[w] : bb;
            nn |= s_nan[w];
        }
        const uint32_t key = nn ? kProdNaN : static_cast<uint32_t>(bb >> 32);
        const uint32_t id = ~static_cast<uint32_t>(bb);
        P.rec[2 * static_cast<size_t>(item) + tid] =
            (static_cast<uint64_t>(P.tag) << 32) | (tid == 0 ? key : id);
    }
}

__global__ __launch_bounds__(kThreads) void k_produce_tokens(ProduceParams P) {
    // one wave per (b, j): lanes read the chunk records in parallel
    const int lane = threadIdx.x & 63;
    const int rj = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (rj >= P.B * P.K) return;
    uint64_t best = 0ull;
    bool ok = true;
    for (int c = lane; c < P.nchp; c += 64) {
        const uint64_t* r = P.rec + 2 * (static_cast<size_t>(rj) * P.nchp + c);
        const uint64_t w0 = r[0], w1 = r[1];
        if (static_cast<uint32_t>(w0 >> 32) != P.tag || static_cast<uint32_t>(w1 >> 32) != P.tag) ok = false;
        const uint64_t pk = (static_cast<uint64_t>(static_cast<uint32_t>(w0)) << 32) |
                            static_cast<uint32_t>(~static_cast<uint32_t>(w1));
        best = pk > best ? pk : best;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(best), off, 64);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(best >> 32), off, 64);
        const uint64_t ob = (static_cast<uint64_t>(hi) << 32) | lo;
        best = ob > best ? ob : best;
    }
    ok = __ballot(!ok) == 0ull;
    const bool nan = static_cast<uint32_t>(best >> 32) == kProdNaN;
    if (lane == 0) P.tokens[rj] = (ok && !nan) ? static_cast<int32_t>(~static_cast<uint32_t>(best)) : -1;
}

hipError_t launch_produce(const ProduceParams& p, int dtype, hipStream_t s, const LaunchEvents& ev) {
    const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(p.B) * p.K * p.nchp);
    if (dtype == DT_BF16)
        hipExtLaunchKernelGGL(k_produce<DT_BF16>, dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, p);
    else
        hipExtLaunchKernelGGL(k_produce<DT_F32>, dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, p);
    return hipGetLastError();
}

hipError_t launch_produce_tokens(const ProduceParams& p, hipStream_t s, const LaunchEvents& ev) {
    const unsigned grid = static_cast<unsigned>((static_cast<int64_t>(p.B) * p.K + kWaves - 1) / kWaves);
    hipExtLaunchKernelGGL(k_produce_tokens, dim3(grid), dim3(kThreads), 0, s, ev.start, ev.stop, 0, p);
    return hipGetLastError();
}

}  // namespace sv
