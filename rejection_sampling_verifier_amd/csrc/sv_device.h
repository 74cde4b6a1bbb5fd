// Device helpers for the verify-step kernels: element formats, wave64
// reductions and scans, the Philox4x32-10 generator, order keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {

#define SV_INF __builtin_huge_valf()

// ---------------------------------------------------------------------------
// Element formats.  A logit row is read as aligned 16-byte vectors: 4 fp32
// or 8 bf16 values.  bf16 widens to fp32 exactly by placing its 16 bits in
// the high half of the word.
// ---------------------------------------------------------------------------
template <int DT> struct Fmt;
template <> struct Fmt<DT_F32> {
    static constexpr int E = 4, VE = 4;
    static constexpr uint32_t NEG_INF_WORD = 0xFF800000u;
};
template <> struct Fmt<DT_BF16> {
    static constexpr int E = 2, VE = 8;
    static constexpr uint32_t NEG_INF_WORD = 0xFF80FF80u;
};

template <int DT> __device__ __forceinline__ void unpack(const uint4& v, float* f);
template <> __device__ __forceinline__ void unpack<DT_F32>(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
}
template <> __device__ __forceinline__ void unpack<DT_BF16>(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xFFFF0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xFFFF0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// 16-byte load through the global address space (global_load_dwordx4, not
// the generic flat path the compiler picks for pointers held in a struct).
typedef unsigned int sv_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const sv_u32x4 sv_g_u32x4;
__device__ __forceinline__ uint4 gload16(const uint4* p) {
    const sv_u32x4 v = *(sv_g_u32x4*)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// The same with the nontemporal hint (data read once).
__device__ __forceinline__ uint4 gload16_nt(const uint4* p) {
    const sv_u32x4 v = __builtin_nontemporal_load((sv_g_u32x4*)(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int DT> __device__ __forceinline__ float load_elem(const uint8_t* row, int64_t i);
template <> __device__ __forceinline__ float load_elem<DT_F32>(const uint8_t* row, int64_t i) {
    return reinterpret_cast<const float*>(row)[i];
}
template <> __device__ __forceinline__ float load_elem<DT_BF16>(const uint8_t* row, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[i]) << 16);
}

// Loads ids [id0, id0 + nv) of a row into f[0..nv), nv <= 8, by 16-byte
// vectors when the run is aligned and whole, by elements otherwise.
template <int DT>
__device__ __forceinline__ void load8(const uint8_t* row, int64_t id0, int nv, float* f) {
    constexpr int E = Fmt<DT>::E, VE = Fmt<DT>::VE;
    const uint8_t* p = row + id0 * E;
    if (nv == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
        const uint4* vp = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int k = 0; k < 8 / VE; ++k) unpack<DT>(gload16(vp + k), f + k * VE);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (i < nv) ? load_elem<DT>(row, id0 + i) : -SV_INF;
    }
}

// Hardware 2^x (v_exp_f32, ~1 ulp).  Arguments below -126 give results
// below 2^-126 relative to the row's largest term, which no decision can see;
// the library's exp2f would spend five more instructions on them.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Temperature-scaled exponent 2^(l*c - o) with c = c_hi + c_lo.  Both fused
// multiply-adds are needed to keep c exact to ~2^-48: a float c alone would
// tilt every distribution by up to 2^-24 relative in the exponent.  c_lo > 0
// keeps l = -inf at -inf (never -inf + inf).
__device__ __forceinline__ float tempexp(float l, float c_hi, float c_lo, float o) {
    return hw_exp2(fmaf(l, c_lo, fmaf(l, c_hi, -o)));
}

// max of three floats in one v_max3_f32 (no canonicalising moves; a NaN
// input is caught later through the sum it poisons).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}


// Order key of a logit: unsigned compare of keys = numeric compare of values
// (-0 and +0 share a key).
__device__ __forceinline__ uint32_t order_key(float l) {
    uint32_t u = __float_as_uint(l + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}
__device__ __forceinline__ bool is_kept(uint32_t key, int64_t id, uint32_t tau, int32_t cut) {
    return key > tau || (key == tau && id <= cut);
}

// ---------------------------------------------------------------------------
// Wave64 reductions and scans.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}
// Inclusive prefix sum over the wave's lanes, fixed order.
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        double t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Wave64 scans and reductions through DPP (data-parallel lane moves inside
// the VALU, no LDS round trip): row_shr 1, 2, 4, 8 scan each row of 16 lanes,
// then row_bcast15 and row_bcast31 carry row totals into the later rows.  A
// lane whose source is outside its row keeps `old`, the operation's identity.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
constexpr int kDppWaveShr1 = 0x138;  // lane i reads lane i-1 across the whole wave

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_int(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, ROWS, 0xF, false);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
// A lane move whose lanes outside the moved range read 0 and whose rows
// outside ROWS are left undefined: for sums that only the group's last lane
// keeps, where no `old` value needs setting first.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_mov_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b), CTRL, ROWS, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), CTRL, ROWS, 0xF, true);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
// Sum over each group of G consecutive lanes (G = 16, 32 or 64, groups
// aligned to G), held by the group's last lane; other lanes hold partial or
// undefined values.
template <int G>
__device__ __forceinline__ double group_sum_dpp(double v) {
    static_assert(G == 16 || G == 32 || G == 64, "rows of 16 lanes");
    v += dpp_mov_f64<kDppRowShr1, 0xF>(v);
    v += dpp_mov_f64<kDppRowShr2, 0xF>(v);
    v += dpp_mov_f64<kDppRowShr4, 0xF>(v);
    v += dpp_mov_f64<kDppRowShr8, 0xF>(v);
    if (G >= 32) v += dpp_mov_f64<kDppRowBcast15, 0xA>(v);
    if (G >= 64) v += dpp_mov_f64<kDppRowBcast31, 0xC>(v);
    return v;
}
// Inclusive prefix sum over the wave's lanes (fixed order of additions).
__device__ __forceinline__ double wave_scan_dpp(double v) {
    v += dpp_f64<kDppRowShr1, 0xF>(v);
    v += dpp_f64<kDppRowShr2, 0xF>(v);
    v += dpp_f64<kDppRowShr4, 0xF>(v);
    v += dpp_f64<kDppRowShr8, 0xF>(v);
    v += dpp_f64<kDppRowBcast15, 0xA>(v);
    v += dpp_f64<kDppRowBcast31, 0xC>(v);
    return v;
}
__device__ __forceinline__ double lane63(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), 63);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
// Lane `l` (wave-uniform) of a double.
__device__ __forceinline__ double readlane_f64(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), l);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), l);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
// Sum over the wave, the same in every lane.
__device__ __forceinline__ double wave_sum_dpp(double v) { return lane63(wave_scan_dpp(v)); }
__device__ __forceinline__ int wave_max_int_dpp(int v) {
    constexpr int lo = static_cast<int>(0x80000000u);
    v = max(v, dpp_int<kDppRowShr1, 0xF>(lo, v));
    v = max(v, dpp_int<kDppRowShr2, 0xF>(lo, v));
    v = max(v, dpp_int<kDppRowShr4, 0xF>(lo, v));
    v = max(v, dpp_int<kDppRowShr8, 0xF>(lo, v));
    v = max(v, dpp_int<kDppRowBcast15, 0xA>(lo, v));
    v = max(v, dpp_int<kDppRowBcast31, 0xC>(lo, v));
    return __builtin_amdgcn_readlane(v, 63);
}
// Maximum over the wave, the same in every lane (-inf is the identity).
__device__ __forceinline__ float wave_max_dpp(float v) {
    constexpr int ninf = static_cast<int>(0xFF800000u);
    v = fmaxf(v, __int_as_float(dpp_int<kDppRowShr1, 0xF>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_int<kDppRowShr2, 0xF>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_int<kDppRowShr4, 0xF>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_int<kDppRowShr8, 0xF>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_int<kDppRowBcast15, 0xA>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_int<kDppRowBcast31, 0xC>(ninf, __float_as_int(v))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_min_int_dpp(int v) {
    constexpr int hi = 0x7FFFFFFF;
    v = min(v, dpp_int<kDppRowShr1, 0xF>(hi, v));
    v = min(v, dpp_int<kDppRowShr2, 0xF>(hi, v));
    v = min(v, dpp_int<kDppRowShr4, 0xF>(hi, v));
    v = min(v, dpp_int<kDppRowShr8, 0xF>(hi, v));
    v = min(v, dpp_int<kDppRowBcast15, 0xA>(hi, v));
    v = min(v, dpp_int<kDppRowBcast31, 0xC>(hi, v));
    return __builtin_amdgcn_readlane(v, 63);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11, section 3.2): per round, 32x32->64
// products of counter words 0 and 2 with 0xD2511F53 and 0xCD9E8D57; output
// (hi2 ^ c1 ^ k0, lo2, hi0 ^ c3 ^ k1, lo0); key bumped by the Weyl constants
// 0x9E3779B9, 0xBB67AE85 between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
        const uint32_t hi2 = __umulhi(0xCD9E8D57u, c.z), lo2 = 0xCD9E8D57u * c.z;
        c = make_uint4(hi2 ^ c.y ^ k0, lo2, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}
// 24-bit uniform in [0, 1 - 2^-24].
__device__ __forceinline__ double word_uniform(uint32_t w) {
    return static_cast<double>(w >> 8) * (1.0 / 16777216.0);
}

}  // namespace sv
