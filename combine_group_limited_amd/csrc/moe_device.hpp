// moe_device.hpp -- device-side helpers shared by the gfx950 kernels.
//
// Wave64 throughout: every helper that exchanges data between lanes assumes a
// full 64-lane wave with all lanes active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgl {

constexpr int kWave = 64;

// Index of the calling wave within its block, as a wave-uniform (scalar)
// value: lets the compiler keep per-wave addresses in SGPRs and use scalar
// loads for per-wave data.
__device__ __forceinline__ int wave_in_block() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Native vector types (usable with the nontemporal load/store builtins).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global loads/stores of streams that are touched once: NT = 1 marks them
// non-temporal (streaming) so they do not displace reusable lines.
template <int NT, typename V>
__device__ __forceinline__ V load_stream(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int NT, typename V>
__device__ __forceinline__ void store_stream(V v, V* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------------------
// fp32 exponential used for router scores.  Router selection must agree bit
// for bit with an independent host implementation, so the recipe is fixed:
//   clamp: z >= 80 -> +inf, z <= -80 -> 0 (keeps every result a normal number)
//   n = rint(z * log2(e));  r = z - n*ln2_hi - n*ln2_lo (two fmas; ln2_hi has
//   17 significant bits so n*ln2_hi is exact)
//   p = sum_{i<=7} r^i/i! by Horner with fma, coefficients rounded to fp32
//   result = p * 2^n (exact, v_ldexp_f32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_fixed(float z) {
    // branch-free: evaluate on the clamped argument, then select the clamp
    // results (identical to returning early for |z| >= 80)
    const float zc = __builtin_fminf(__builtin_fmaxf(z, -80.0f), 80.0f);
    const float n = __builtin_rintf(zc * 1.44269504f);
    float r = __builtin_fmaf(-n, 0x1.62e4p-1f, zc);
    r = __builtin_fmaf(-n, 1.4286068e-6f, r);
    float p = 0x1.a01a02p-13f;                 // 1/5040
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f); // 1/720
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);  // 1/120
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);  // 1/24
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);  // 1/6
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float e = __builtin_ldexpf(p, (int)n);
    return (z >= 80.0f) ? __builtin_inff() : ((z <= -80.0f) ? 0.0f : e);
}

__device__ __forceinline__ float sigmoid_fixed(float x) {
    const float e = exp_fixed(-x);
    return 1.0f / (1.0f + e);  // IEEE division (the library is compiled without fast-math)
}

// ---------------------------------------------------------------------------
// Ordering keys: larger key = ranks first.  High word: the score's fp32 bits
// mapped to an unsigned order (-0 folded onto +0 so they compare equal); low
// word: ~index so that among equal scores the lower index wins.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_order(float v) {
    uint32_t b = __float_as_uint(v + 0.0f);          // -0 + 0 = +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float order_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float v, uint32_t index) {
    return ((uint64_t)float_order(v) << 32) | (uint64_t)(0xFFFFFFFFu - index);
}

__device__ __forceinline__ uint32_t key_index(uint64_t k) {
    return 0xFFFFFFFFu - (uint32_t)k;
}

__device__ __forceinline__ float key_value(uint64_t k) {
    return order_float((uint32_t)(k >> 32));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// DPP lane exchange of a 32-bit value within rows of 16 lanes.
//   0xB1 quad_perm[1,0,3,2] (lane ^ 1)    0x4E quad_perm[2,3,0,1] (lane ^ 2)
//   0x141 row_half_mirror (i <-> 7-i)     0x140 row_mirror (i <-> 15-i)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const uint32_t lo = dpp32<CTRL>((uint32_t)v);
    const uint32_t hi = dpp32<CTRL>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t bperm32(uint32_t v, int src_lane) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

__device__ __forceinline__ uint64_t bperm64(uint64_t v, int src_lane) {
    return ((uint64_t)bperm32((uint32_t)(v >> 32), src_lane) << 32) | bperm32((uint32_t)v, src_lane);
}

// Max over aligned segments of W lanes (W a power of two <= 64); every lane of
// a segment receives the segment's maximum.  Within a row (W <= 16) each step
// pairs every lane with a lane of the other half of its current sub-segment.
template <int W>
__device__ __forceinline__ uint64_t seg_max64(uint64_t v) {
    if constexpr (W >= 2) v = umax64(v, dpp64<0xB1>(v));
    if constexpr (W >= 4) v = umax64(v, dpp64<0x4E>(v));
    if constexpr (W >= 8) v = umax64(v, dpp64<0x141>(v));
    if constexpr (W >= 16) v = umax64(v, dpp64<0x140>(v));
    const int lane = (int)__lane_id();
    if constexpr (W >= 32) v = umax64(v, bperm64(v, lane ^ 16));
    if constexpr (W >= 64) v = umax64(v, bperm64(v, lane ^ 32));
    return v;
}

// Max over the whole wave, returned as a wave-uniform value.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
    v = seg_max64<16>(v);
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    uint64_t r = 0;
#pragma unroll
    for (int row = 0; row < 4; ++row) {
        const uint64_t rv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, row * 16) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)lo, row * 16);
        r = umax64(r, rv);
    }
    return r;
}

// Max of non-negative 32-bit values over each row of 16 lanes (all lanes of
// the row receive it).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, dpp32<0xB1>(v));
    v = max(v, dpp32<0x4E>(v));
    v = max(v, dpp32<0x141>(v));
    v = max(v, dpp32<0x140>(v));
    return v;
}

// DPP exchange of a float within rows of 16 lanes (same controls as dpp32).
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max of floats over aligned segments of W lanes (W a power of two <= 64);
// every lane of a segment receives it.  Inputs are finite or -inf.
template <int W>
__device__ __forceinline__ float seg_maxf(float v) {
    if constexpr (W >= 2) v = __builtin_fmaxf(v, dppf<0xB1>(v));
    if constexpr (W >= 4) v = __builtin_fmaxf(v, dppf<0x4E>(v));
    if constexpr (W >= 8) v = __builtin_fmaxf(v, dppf<0x141>(v));
    if constexpr (W >= 16) v = __builtin_fmaxf(v, dppf<0x140>(v));
    const int lane = (int)__lane_id();
    if constexpr (W >= 32) v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, __float_as_int(v))));
    if constexpr (W >= 64) v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v))));
    return v;
}

// Min of unsigned values over aligned segments of W lanes.
template <int W>
__device__ __forceinline__ uint32_t seg_minu(uint32_t v) {
    if constexpr (W >= 2) v = min(v, dpp32<0xB1>(v));
    if constexpr (W >= 4) v = min(v, dpp32<0x4E>(v));
    if constexpr (W >= 8) v = min(v, dpp32<0x141>(v));
    if constexpr (W >= 16) v = min(v, dpp32<0x140>(v));
    const int lane = (int)__lane_id();
    if constexpr (W >= 32) v = min(v, bperm32(v, lane ^ 16));
    if constexpr (W >= 64) v = min(v, bperm32(v, lane ^ 32));
    return v;
}

// Max of unsigned values over aligned segments of W lanes (W a power of two
// <= 16 uses only DPP; 32 and 64 add permutes).
template <int W>
__device__ __forceinline__ uint32_t seg_maxu(uint32_t v) {
    if constexpr (W >= 2) v = max(v, dpp32<0xB1>(v));
    if constexpr (W >= 4) v = max(v, dpp32<0x4E>(v));
    if constexpr (W >= 8) v = max(v, dpp32<0x141>(v));
    if constexpr (W >= 16) v = max(v, dpp32<0x140>(v));
    const int lane = (int)__lane_id();
    if constexpr (W >= 32) v = max(v, bperm32(v, lane ^ 16));
    if constexpr (W >= 64) v = max(v, bperm32(v, lane ^ 32));
    return v;
}

// Max of unsigned values over the whole wave, as a wave-uniform value: DPP
// inside rows of 16, then the four row results on the scalar unit.
__device__ __forceinline__ uint32_t wave_maxu(uint32_t v) {
    v = seg_maxu<16>(v);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// Max of floats over the whole wave, as a wave-uniform value.
__device__ __forceinline__ float wave_maxf(float v) {
    v = seg_maxf<16>(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two bf16 (round to nearest even), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo;
    const __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Four fp32 -> four OCP E4M3FN codes (round to nearest even), byte i = input i.
// Inputs are first clamped to [-448, 448] so magnitudes above the largest
// finite code saturate instead of becoming NaN; the clamp keeps -0.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}


// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their "no wait" maxima):
// on CDNA the vector-memory counter also counts outstanding stores.
constexpr int kWaitStores = 0x0F70;

// ---------------------------------------------------------------------------
// FP8 quantisation of one 512-channel unit held as 8 bf16 per lane (lane l:
// channels 8l..8l+7), so a 128-channel scale block is one 16-lane DPP row.
// ---------------------------------------------------------------------------
// absmax of the 8 bf16 values held by a lane, as a 15-bit magnitude pattern
__device__ __forceinline__ uint32_t lane_absmax_bits(const u32x4& v) {
    const uint32_t m0 = max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu);
    const uint32_t m1 = max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu);
    const uint32_t m2 = max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu);
    const uint32_t m3 = max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu);
    return max(max(m0, m1), max(m2, m3));
}

// Block scale of a 128-channel block with absmax aa (> 0).  POW2 = false: scale = a/448, inv = 448/a (IEEE divisions).
// POW2 = true: scale = 2^e with e the smallest integer such that a <= 448*2^e;
// writing a = m * 2^E (m in [1,2)) and 448 = 1.75 * 2^8 gives
// e = E - 8 + (m > 1.75), read straight off a's bits, and inv = 2^-e exactly.
template <bool POW2>
__device__ __forceinline__ void block_scale(float aa, float& scale, float& inv) {
    if constexpr (POW2) {
        const uint32_t b = __float_as_uint(aa);
        const int e = (int)(b >> 23) - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
        scale = __uint_as_float((uint32_t)(e + 127) << 23);
        inv = __uint_as_float((uint32_t)(127 - e) << 23);
    } else {
        scale = aa / 448.0f;
        inv = 448.0f / aa;
    }
}

// Codes (8 per lane, byte i = channel 8l+i) and the scale of the lane's
// 128-channel block: amax floored at 2^-100, codes of x * inv.
template <bool POW2>
__device__ __forceinline__ u32x2 quantize_unit(const u32x4& v, float& scale) {
    const uint32_t m = row16_max_u32(lane_absmax_bits(v));
    const float amax = __uint_as_float(m << 16);
    const float aa = amax > 0x1p-100f ? amax : 0x1p-100f;
    float inv;
    block_scale<POW2>(aa, scale, inv);
    u32x2 code;
    code.x = pack_e4m3x4(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
    code.y = pack_e4m3x4(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
    return code;
}

// Sum over the wave (DPP inside rows of 16, the four row sums on the scalar
// unit), returned in every lane.
__device__ __forceinline__ int wave_sum(int v) {
    v += (int)dpp32<0xB1>((uint32_t)v);
    v += (int)dpp32<0x4E>((uint32_t)v);
    v += (int)dpp32<0x141>((uint32_t)v);
    v += (int)dpp32<0x140>((uint32_t)v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
           __builtin_amdgcn_readlane(v, 48);
}

// Inclusive scan of one value per lane across a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive scan of tot[0..E) (each rounded up to a multiple of A when A > 1)
// into off[0..E] (off[E] = total), by a whole block of THREADS threads: each
// thread owns a run of ceil(E/THREADS) experts.  Both arrays may be in LDS.
template <int THREADS>
__device__ void block_exclusive_scan(const int32_t* tot, int32_t* off, int E, int A) {
    constexpr int kWaves = THREADS / kWave;
    __shared__ int32_t wave_tot[kWaves];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int per = (E + THREADS - 1) / THREADS;
    const int lo = min(tid * per, E), hi = min(lo + per, E);
    auto span = [A](int c) { return A > 1 ? (c + A - 1) / A * A : c; };
    int s = 0;
    for (int e = lo; e < hi; ++e) s += span(tot[e]);
    const int inc = wave_inclusive_scan(s);
    if (lane == 63) wave_tot[w] = inc;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q)
        if (q < w) base += wave_tot[q];
    int run = base + inc - s;
    for (int e = lo; e < hi; ++e) {
        off[e] = run;
        run += span(tot[e]);
    }
    if (tid == THREADS - 1) off[E] = run;
    __syncthreads();
}

}  // namespace cgl
