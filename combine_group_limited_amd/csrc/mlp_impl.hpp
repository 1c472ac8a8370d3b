// mlp_impl.hpp -- the block body of the expert-MLP GEMMs and the host-side
// tile and LDS arithmetic, shared by the standalone up/down launches
// (mlp.hip, which also says which pages this follows and how the tiles and
// the K loop work) and the one-launch MoE layer (layer.hip).
#pragma once
#include "moe_device.hpp"

namespace cgl {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;    // K per scale block = K per LDS stage
constexpr int kBR = 256;    // weight rows per block tile
constexpr int kActN = 128;  // up: act columns per block (128 gate + 128 up weight rows)
constexpr int kThreads = 256;

// s_waitcnt vmcnt(N) (6-bit count split over bits 3:0 and 15:14), with
// expcnt at its "no wait" maximum and lgkmcnt either at its maximum (LGKM =
// false) or 0
template <int N, bool LGKM = false>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((LGKM ? 0x0070 : 0x0F70) | (N & 15) | ((N >> 4) << 14));
}

template <int TM>
struct Tile {
    static constexpr int kBM = 64 * TM;                    // rows per block
    static constexpr int kStageBytes = (kBM + kBR) * kBK;  // A stage, then B stage
    static constexpr int kCopies = (kBM + kBR) / 8 / 4;    // 1 KiB copies per wave per stage
};

struct MlpArgs {
    const uint8_t* a;      // [N, K] codes
    const float* as;       // [N, K/128] powers of two
    const uint8_t* w;      // [E, WR, K] codes
    const float* ws;       // [E, WR/128, K/128] powers of two
    const int32_t* cnt_e;  // [E]
    const int32_t* off_e;  // [E+1]
    uint8_t* act;          // up: [N, I] codes
    float* act_s;          // up: [N, I/128]
    uint16_t* y;           // down: [N, WR] bf16
    int N, K, WR, E, C, I;
    int gx, rw, rh, nrect;  // tile grid width (column tiles) and the XCD rectangles
};

__device__ __forceinline__ uint32_t e8m0(float s) { return (__float_as_uint(s) >> 23) & 0xFFu; }

__device__ __forceinline__ int rows_of(const MlpArgs& a, int e, int& start) {
    int cnt = a.cnt_e[e];
    cnt = cnt < 0 ? 0 : cnt;
    if (a.C > 0) {
        start = e * a.C;
        cnt = cnt < a.C ? cnt : a.C;
    } else {
        start = a.off_e[e];
    }
    if (start < 0 || (long long)start + cnt > a.N) cnt = 0;  // inconsistent layout: skip
    return cnt;
}

// XOR swizzle of the 16-byte chunks of a 128-byte-row stage.  A 16-byte LDS
// read is served 16 lanes at a time from 64 four-byte banks (256 bytes); 16
// lanes read 16 consecutive rows at one logical chunk, rows of equal parity
// share a 128-byte bank half, and the key (r >> 1) & 7 gives the eight rows
// of each parity distinct chunks, so the 16 reads hit distinct banks.
__device__ __forceinline__ int swz_key(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz(int r, int c) { return r * kBK + ((c ^ swz_key(r)) << 4); }

// Row-scale word of K block kb for wave row / lane slot w (0..63).
__device__ __forceinline__ int sc_word(int kb, int w) { return kb * 64 + w; }

// Weight row (within the expert's [WR, K] matrix) staged at B-stage row r.
template <bool UP>
__device__ __forceinline__ int wrow_of(const MlpArgs& a, int n0, int r) {
    if constexpr (UP) return r < kActN ? n0 + r : a.I + n0 + (r - kActN);
    const int w = n0 + r;
    return w < a.WR ? w : a.WR - 1;
}

__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Max of non-negative 32-bit values over each half-wave (lanes 0-31, 32-63).
__device__ __forceinline__ uint32_t half32_max_u32(uint32_t v) {
    v = row16_max_u32(v);
    return max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
}

// One scaled 32x32x64 MFMA; OA and OB pick the scale bytes.
template <int OA, int OB>
__device__ __forceinline__ f32x16 mfma32(const i32x8& a, const i32x8& b, const f32x16& c, uint32_t sa, uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, (int)sa, OB, (int)sb);
}

template <int TM>
struct Frag {
    i32x8 a[TM];
    i32x8 b[4];
    uint32_t sa, sb;
};

template <bool UP, int TM, int T, int U>
__device__ __forceinline__ void mma_tile(f32x16 (&acc)[TM][4], const Frag<TM>& f) {
    // op_sel picks byte T of the A scales and, for up, byte 0 (gate) or 1
    // (up) of the weight scales
    acc[T][U] = mfma32<T, (UP && U >= 2) ? 1 : 0>(f.a[T], f.b[U], acc[T][U], f.sa, f.sb);
    if constexpr (U + 1 < 4) mma_tile<UP, TM, T, U + 1>(acc, f);
    else if constexpr (T + 1 < TM) mma_tile<UP, TM, T + 1, 0>(acc, f);
}

// NR: stage buffers in the ring (2, or 3 for 128-row tiles when it fits:
// their stages are smaller and the kernel streams weights, so a second stage
// in flight pays).
// FRESH: called once per tile from a persistent loop; the thread index is
// re-read opaquely per tile, so that nothing derived from it is hoisted out
// of the loop and kept live across the whole K loop (which makes the
// 256-row kernel spill).
template <bool UP, int TM, int NR, bool FRESH = false>
__device__ __forceinline__ void mlp_block(const MlpArgs& a, int blk) {
    using TL = Tile<TM>;
    constexpr int kBM = TL::kBM, kStageBytes = TL::kStageBytes, kCopies = TL::kCopies;
    constexpr int kSW = TM > 2 ? 4 : 2;  // bytes per row-scale word (one byte per row tile)
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* ring = smem;                                          // [NR][kStageBytes]
    const int KB = a.K / kBK;
    uint8_t* a_sc = smem + NR * kStageBytes;                       // [KB][64] words: byte t = row tile t
    uint32_t* w_sc = (uint32_t*)(a_sc + KB * 64 * kSW);            // [KB][2]
    int32_t* tot = (int32_t*)(w_sc + 2 * KB);                      // [E]
    int32_t* tpref = tot + a.E;                                    // [E+1]

    int tid = threadIdx.x;
    if (FRESH) asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;
    const int m = lane & 31, g = lane >> 5;

    // Tile order: the chip deals consecutive blocks to its 8 XCDs in turn and
    // each XCD has its own L2, so the 32 blocks an XCD runs at once are given
    // one rh x rw rectangle of (row slot, column) tiles: 4 x 8 for up shares
    // each A panel among 8 blocks and each weight panel among 4 in one L2.
    int slot, col;
    {
        const int b = blk, x = b & 7, i = b >> 3;
        const int R = (i >> 5) * 8 + x, p = i & 31;
        if (R >= a.nrect) return;  // block-uniform
        const int rpr = a.gx / a.rw;  // rectangles per rectangle row
        slot = (R / rpr) * a.rh + p / a.rw;
        col = (R % rpr) * a.rw + p % a.rw;
    }

    // ---- which expert and row tile this block computes --------------------
    for (int e = tid; e < a.E; e += kThreads) {
        int st;
        tot[e] = (rows_of(a, e, st) + kBM - 1) / kBM;
    }
    __syncthreads();
    block_exclusive_scan<kThreads>(tot, tpref, a.E, 0);  // ends with a barrier
    if (slot >= tpref[a.E]) return;  // block-uniform
    int lo = 0, hi = a.E - 1;        // the expert e with tpref[e] <= slot < tpref[e+1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tpref[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    int start;
    const int cnt = rows_of(a, e, start);
    const int row0 = start + (slot - tpref[e]) * kBM;
    const int nvalid = min(kBM, start + cnt - row0);
    const int n0 = col * (UP ? kActN : kBR);

    // ---- K loop -----------------------------------------------------------
    // One 128-deep stage (kBM rows of A and 256 weight rows, 128 bytes each)
    // goes to LDS by direct global->LDS copies: each instruction moves 1 KiB
    // (8 rows) with lane i filling LDS bytes [16i, 16i+16), so lane i fetches
    // the logical chunk that the swizzle puts at that position.  Each copy's
    // rows are all A rows or all weight rows, so it takes a wave-uniform base
    // and a 32-bit row offset.  Whole 128-byte lines per row matter: the same
    // traffic in 64-byte halves moves 25 % slower into the CUs.
    const uint8_t* wbase = a.w + (size_t)e * a.WR * a.K;
    const int wv = FRESH ? __builtin_amdgcn_readfirstlane(tid >> 6) : wave_in_block();  // w, as a scalar
    const int rl = lane >> 3;        // row within the 8-row group
    uint32_t coff[kCopies];
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
        const int q = wv * kCopies + j, r = 8 * q + rl;
        const int row = r < kBM ? min(row0 + r, a.N - 1) : wrow_of<UP>(a, n0, r - kBM);
        const int lc = (lane & 7) ^ swz_key(r);  // logical chunk held at this lane's position
        coff[j] = (uint32_t)row * (uint32_t)a.K + (uint32_t)(lc * 16);
    }
    // Stages past the end are replaced by copies of one line that nobody
    // reads, so the loop needs no branch around its copies.
    auto issue = [&](int st, int buf) {
        uint8_t* d = ring + buf * kStageBytes;
        const bool real = st < KB;
        const uint32_t kof = real ? (uint32_t)(st * kBK) : 0u;
#pragma unroll
        for (int j = 0; j < kCopies; ++j) {
            const int q = wv * kCopies + j;
            const uint8_t* base = 8 * q < kBM ? a.a : wbase;
            const uint32_t off = real ? coff[j] + kof : 0u;
            __builtin_amdgcn_global_load_lds((const void*)(base + off),
                                             (__attribute__((address_space(3))) void*)(d + q * 1024), 16, 0, 0);
        }
    };

    // Fragments of one 64-deep half of a stage: TM row tiles of A and 4
    // weight tiles, 32 bytes per lane each (chunks 4h + 2g and 4h + 2g + 1 of
    // the lane's row), and the stage's scales.
    const int arow0 = 32 * TM * wr + m;
    int brow[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if constexpr (UP) brow[u] = (u < 2 ? 0 : kActN) + 64 * wc + 32 * (u & 1) + m;
        else brow[u] = 128 * wc + 32 * u + m;
    }
    auto read = [&](Frag<TM>& f, int st, int buf, int h) {
        const uint8_t* sA = ring + buf * kStageBytes;
        const uint8_t* sB = sA + kBM * kBK;
        const int c0 = 4 * h + 2 * g;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int row = arow0 + 32 * t;
            const i32x4 lo4 = *(const i32x4*)(sA + swz(row, c0));
            const i32x4 hi4 = *(const i32x4*)(sA + swz(row, c0 + 1));
            f.a[t] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const i32x4 lo4 = *(const i32x4*)(sB + swz(brow[u], c0));
            const i32x4 hi4 = *(const i32x4*)(sB + swz(brow[u], c0 + 1));
            f.b[u] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        const int wi = sc_word(st, wr * 32 + m);
        if constexpr (kSW == 4) f.sa = ((const uint32_t*)a_sc)[wi];
        else f.sa = ((const uint16_t*)a_sc)[wi];
        f.sb = w_sc[st * 2 + wc];
    };

    f32x16 acc[TM][4];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][u][i] = 0.0f;

    // Stage protocol (NR buffers; stage S lives in buffer S % NR).  Each
    // stage is two MFMA halves.  During half 0 of S the wave reads the
    // fragments of half 1 of S; then every wave waits until its copies of
    // stage S+1 have landed (only the NR - 2 later stages may still be in
    // flight; s_waitcnt vmcnt counts copies in issue order) and its own reads
    // are done, and meets the others at a bare barrier: S+1 is now visible to
    // all and buffer S % NR is free, so stage S+NR is issued into it, and
    // half 1 of S runs while half 0 of S+1 is read.  One barrier per stage; a
    // stage's copies have NR - 1 stages of MFMAs to land.
    Frag<TM> f0, f1;

    // ---- scales of the whole K range, as E8M0 bytes ------------------------
    // a_sc word sc_word(kb, 32 wr + m) (kSW bytes) holds the scales of rows
    // 32*TM*wr + 32t + m (t < TM) in byte t.  The block's kBM x KB row scales are one
    // contiguous run of a.as (reads past the array's end take its last
    // element: those rows are never stored).  Their loads are issued before
    // the first stages' copies: s_waitcnt vmcnt retires loads in issue order,
    // so scale loads issued behind 128 KiB of copies would wait for all of
    // them.  With KB a multiple of 4 and a 16-byte aligned run, sixteen
    // 16-byte loads per thread cover 64 Ki scales per batch (K <= 32768 at
    // 256-row tiles: one batch); otherwise single scales, sixteen at a time.
    auto a_sc_put = [&](int r, int kb, float v) {
        a_sc[sc_word(kb, (r / (32 * TM)) * 32 + (r & 31)) * kSW + (r / 32) % TM] = (uint8_t)e8m0(v);
    };
    const int n_sc = kBM * KB;
    const float* src_sc = a.as + (size_t)row0 * KB;
    const int last_sc = min(n_sc, (a.N - row0) * KB) - 1;
    const bool vec_sc = (KB & 3) == 0 && ((reinterpret_cast<uintptr_t>(src_sc) & 15) == 0);
    constexpr int kSV = 16;  // 16-byte scale loads per thread per batch
    f32x4 sv[kSV];
    if (vec_sc) {
#pragma unroll
        for (int j = 0; j < kSV; ++j) sv[j] = ((const f32x4*)src_sc)[min(tid + j * kThreads, last_sc >> 2)];
    }
    const int WRB = a.WR / kBK;
    auto w_sc_load = [&](int i) -> uint32_t {
        const int kb = i >> 1, which = i & 1;
        if constexpr (UP) {  // byte 0 the gate block, byte 1 the up block (both wave columns)
            const size_t base = (size_t)e * WRB * KB + kb;
            return e8m0(a.ws[base + (size_t)(n0 / kBK) * KB]) | (e8m0(a.ws[base + (size_t)((a.I + n0) / kBK) * KB]) << 8);
        } else {             // the wave column's 128 output rows
            const int blk = min(n0 / kBK + which, WRB - 1);
            return e8m0(a.ws[((size_t)e * WRB + blk) * KB + kb]);
        }
    };
    float ws_raw0 = 0.0f, ws_raw1 = 0.0f;  // this thread's first w_sc entry, loaded early
    if (tid < 2 * KB) {
        const int kb = tid >> 1, which = tid & 1;
        if constexpr (UP) {
            const size_t base = (size_t)e * WRB * KB + kb;
            ws_raw0 = a.ws[base + (size_t)(n0 / kBK) * KB];
            ws_raw1 = a.ws[base + (size_t)((a.I + n0) / kBK) * KB];
        } else {
            ws_raw0 = a.ws[((size_t)e * WRB + min(n0 / kBK + which, WRB - 1)) * KB + kb];
        }
    }

#pragma unroll
    for (int q = 0; q < NR; ++q) issue(q, q);

    if (vec_sc) {
        // float4 f of the run holds scales 4f..4f+3: one row, four K blocks
        for (int j0 = 0; j0 * kThreads * 4 < n_sc; j0 += kSV) {
            if (j0 > 0) {
#pragma unroll
                for (int j = 0; j < kSV; ++j) sv[j] = ((const f32x4*)src_sc)[min(tid + (j0 + j) * kThreads, last_sc >> 2)];
            }
#pragma unroll
            for (int j = 0; j < kSV; ++j) {
                const int f4 = tid + (j0 + j) * kThreads;
                if (4 * f4 < n_sc) {
                    const int r = (4 * f4) / KB, kb = 4 * f4 - r * KB;
#pragma unroll
                    for (int c = 0; c < 4; ++c) a_sc_put(r, kb + c, sv[j][c]);
                }
            }
        }
    } else {
        // thread i takes elements i, i + 256, ...; (row, kb) is stepped
        const int dq = kThreads / KB, dr = kThreads - dq * KB;
        int r = tid / KB, kb = tid - r * KB;
        for (int j0 = 0; j0 * kThreads < n_sc; j0 += 16) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = src_sc[min(tid + (j0 + j) * kThreads, last_sc)];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (tid + (j0 + j) * kThreads < n_sc) a_sc_put(r, kb, v[j]);
                r += dq;
                kb += dr;
                if (kb >= KB) {
                    kb -= KB;
                    ++r;
                }
            }
        }
    }
    if (tid < 2 * KB) {
        if constexpr (UP) w_sc[tid] = e8m0(ws_raw0) | (e8m0(ws_raw1) << 8);
        else w_sc[tid] = e8m0(ws_raw0);
    }
    for (int i = tid + kThreads; i < 2 * KB; i += kThreads) w_sc[i] = w_sc_load(i);
    __syncthreads();  // scales in LDS
    // stage 0 has landed (the later stages' copies may still be in flight:
    // every other load was consumed above, and the loop waits for stage 1)
    wait_vm<(NR - 1) * kCopies>();
    bare_barrier();
    read(f0, 0, 0, 0);

    constexpr int kM = 4 * TM;
    constexpr int kDs = (2 * (TM + 4) + 2 + kM - 1) / kM;  // LDS reads per MFMA slot
    constexpr int kVm = (kCopies + kM - 1) / kM;           // copies per MFMA slot
    int st = 0;
    for (; st + 1 < KB; ++st) {
        const int b = st % NR;
        read(f1, st, b, 1);
        mma_tile<UP, TM, 0, 0>(acc, f0);
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);  // LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<(NR - 2) * kCopies, true>();
        bare_barrier();
        issue(st + NR, b);
        read(f0, st + 1, (st + 1) % NR, 0);
        mma_tile<UP, TM, 0, 0>(acc, f1);
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, kVm, 0);  // global->LDS copies
            __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);  // LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // the last stage (kept in program order: interleaving its two halves
    // with each other and the epilogue makes the register allocator spill)
    read(f1, st, st % NR, 1);
    mma_tile<UP, TM, 0, 0>(acc, f0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<0, true>();
    mma_tile<UP, TM, 0, 0>(acc, f1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // every copy has landed (waited above); the ring is reused below


    if constexpr (UP) {
        // ---- SwiGLU into an fp32 LDS tile, then one thread per row: row amax
        // over the block's 128 act columns, power-of-two scale, FP8 codes ----
        // The lane holds, for row tile t and element i, row 32*TM*wr + 32t +
        // 8(i/4) + 4g + i%4 at act column 64wc + 32u + m (u = 0, 1), so four
        // consecutive elements are four consecutive rows of one column: the
        // tile is column-major with columns padded to kBM + 4 floats (16-byte
        // stores, lanes of a row group on distinct banks).  SwiGLU uses the
        // hardware exp2 and reciprocal (1 ulp each; relative error below
        // |g|*2^-24 + 2^-21 for the gate value g).
        constexpr int kCS = kBM + 4;
        float* ft = (float*)ring;  // [128][kCS]
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float gg = acc[t][u][4 * k + j], uu = acc[t][u + 2][4 * k + j];
                        v[j] = gg * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gg * -1.44269504f)) * uu;
                    }
                    const int row = 32 * TM * wr + 32 * t + 8 * k + 4 * g, col = 64 * wc + 32 * u + m;
                    *(f32x4*)(ft + col * kCS + row) = v;
                }
        __syncthreads();
        if (tid < kBM && tid < nvalid) {
            // the row's 128 values are read once into registers (up to 15
            // LDS reads in flight per wave), then reduced and encoded
            const int r = tid;
            float v[kActN];
#pragma unroll
            for (int c = 0; c < kActN; ++c) v[c] = ft[c * kCS + r];
            uint32_t mx = 0;
#pragma unroll
            for (int c = 0; c < kActN; ++c) mx = max(mx, __float_as_uint(v[c]) & 0x7FFFFFFFu);
            const float amax = __uint_as_float(mx);
            float scale, inv;
            block_scale<true>(amax > 0x1p-100f ? amax : 0x1p-100f, scale, inv);
            uint8_t* dst = a.act + (size_t)(row0 + r) * a.I + n0;
#pragma unroll
            for (int c0 = 0; c0 < kActN; c0 += 16) {
                u32x4 q;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float* p = v + c0 + 4 * j;
                    q[j] = pack_e4m3x4(p[0] * inv, p[1] * inv, p[2] * inv, p[3] * inv);
                }
                *(u32x4*)(dst + c0) = q;
            }
            a.act_s[(size_t)(row0 + r) * (a.I / kBK) + n0 / kBK] = scale;
        }
    } else {
        // ---- BF16 output tile [kBM][256 + 8], staged for 16-byte stores ------
        // (the tile may run into the scale area, which is no longer needed)
        constexpr int kTS = kBR + 8;
        uint16_t* tile = (uint16_t*)ring;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 32 * TM * wr + 32 * t + 8 * (i >> 2) + 4 * g + (i & 3);
                    const int col = 128 * wc + 32 * u + m;
                    const __bf16 b = (__bf16)acc[t][u][i];
                    tile[row * kTS + col] = __builtin_bit_cast(uint16_t, b);
                }
        __syncthreads();
        // streaming stores: the 2H-byte rows are read once, by combine, and
        // would otherwise evict operand panels that other blocks still use
        // (measured: 512 against 557 us at 8 experts x 4096 rows; the up
        // kernel's act rows, read next by this kernel, stay cached)
        for (int i = tid; i < kBM * 32; i += kThreads) {
            const int r = i >> 5, c = i & 31;
            const int col = n0 + c * 8;
            if (r < nvalid && col < a.WR)
                __builtin_nontemporal_store(*(const u32x4*)(tile + r * kTS + c * 8),
                                            (u32x4*)(a.y + (size_t)(row0 + r) * a.WR + col));
        }
    }
}

// Dynamic LDS: the ring, the scales and the tile prefix; at least the
// epilogue's staging tile, which reuses the same bytes from the start.
template <int TM>
size_t lds_bytes_for(int K, int E, int nr) {
    using TL = Tile<TM>;
    const size_t KB = (size_t)K / kBK, sw = TM > 2 ? 4 : 2;
    const size_t loop = nr * (size_t)TL::kStageBytes + KB * 64 * sw + 4 * (2 * KB) + 4 * (2 * (size_t)E + 1);
    const size_t up_tile = (size_t)kActN * (TL::kBM + 4) * 4;
    const size_t down_tile = (size_t)TL::kBM * (kBR + 8) * 2;
    const size_t r = loop > up_tile ? loop : up_tile;
    return r > down_tile ? r : down_tile;
}

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// 256-row tiles when experts average at least 512 rows, else 128-row tiles.
// (64-row tiles for decode-sized batches, to bring more CUs to the weight
// stream, were measured slower: each weight panel then enters two CUs.)
int pick_tm(int N, int E) { return (long long)N >= 512LL * E ? 4 : 2; }
// three stage buffers for 128-row tiles when they fit, else two
int pick_nr(int tm, int K, int E) { return tm == 2 && lds_bytes_for<2>(K, E, 3) <= kMaxLds ? 3 : 2; }


// Fills the tile grid of a launch (column tiles, XCD rectangles) and returns
// the number of blocks: every rectangle gets its 32 blocks, 8 rectangles (one
// per XCD) at a time.
template <bool UP, int TM>
unsigned mlp_grid(MlpArgs& g) {
    g.gx = UP ? g.I / kActN : (g.WR + kBR - 1) / kBR;
    const int gy = g.N / Tile<TM>::kBM + g.E;  // >= sum over experts of ceil(rows / BM)
    if (g.gx == 0 || gy == 0) return 0;
    g.rw = g.gx % 8 == 0 ? 8 : g.gx % 4 == 0 ? 4 : g.gx % 2 == 0 ? 2 : 1;
    g.rh = 32 / g.rw;
    g.nrect = (gy + g.rh - 1) / g.rh * (g.gx / g.rw);
    return (unsigned)((g.nrect + 7) / 8 * 8 * 32);
}

}  // namespace
}  // namespace cgl
