// mlp.hip -- the expert MLP between dispatch and combine, as grouped FP8 GEMMs
// on the gfx950 matrix cores.
//
// Follows the Mega MoE news page (a MoE layer runs dispatch, a first linear
// layer, SwiGLU, a second linear layer and combine; fusing steps removes the
// round trips through memory between them) and the TileKernels news page,
// "functions" (SwiGLU fused with FP8 quantisation): the SwiGLU and the FP8
// requantisation of its output are fused into the first GEMM's epilogue, so
// the 2I-wide pre-activation never reaches memory.
//
// Operands are OCP E4M3FN with power-of-two block scales -- activations one
// per row and 128 columns (as dispatch's FP8_E4M3_POW2 writes them), weights
// one per 128x128 block -- so each 128-deep step is one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 output tile with both scales
// handed to the instruction as E8M0 exponents: no rescaling on the vector
// units.  Operand lane layout of the instruction (measured): lane l holds
// row l%16 and K bytes [16g, 16g+16) and [64+16g, 64+16g+16), g = l/16; the
// E8M0 scale of (row m, 32-deep K block q) is taken from lane 16q+m, so with
// 128-deep scale blocks every lane passes its own row's scale; accumulator
// element i of lane l is row 4g+i, column l%16.
//
// Tiles: a block of 2*WM waves owns BM = 64*WM rows of one expert x 256
// weight rows (up: 128 gate rows and the matching 128 up rows; down: 256
// output columns); wave (wr, wc) owns 64 rows x 128 weight rows = 4 x 8 MFMA
// tiles.  WM = 4 (256 rows, 8 waves, two waves per SIMD) for experts with
// many rows; WM = 2 (128 rows, 4 waves) otherwise.  The K loop stages
// 128-deep slices of both operands in LDS (three stages of 48 KiB for WM = 2,
// two of 64 KiB for WM = 4), filled by direct global->LDS copies issued one
// or two slices ahead; 16-byte chunks are XOR-swizzled by row so fragment
// reads are conflict-free.  Expert row ranges come from the layout (off_e and
// cnt_e, or e*C and min(cnt_e, C) when padded); each block finds its
// (expert, row tile) from the per-expert tile counts, so the grid is sized
// without reading anything back to the host.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;    // K per step (one scale block)
constexpr int kBR = 256;    // weight rows per block tile
constexpr int kActN = 128;  // up: act columns per block (128 gate + 128 up weight rows)

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt at their "no wait" maxima
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

template <int WM>
struct Tile {
    static constexpr int kWaves = 2 * WM;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBM = 64 * WM;                    // rows per block
    static constexpr int kStageBytes = (kBM + kBR) * kBK;  // A slice, then B slice
    static constexpr int kStages = WM == 2 ? 3 : 2;
    static constexpr int kCopiesA = kBM / 8 / kWaves;      // 1 KiB copies per wave per slice
    static constexpr int kCopiesB = kBR / 8 / kWaves;
    static constexpr int kCopies = kCopiesA + kCopiesB;
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
};

__device__ __forceinline__ int e8m0(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFFu); }

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

// LDS offset of 16-byte chunk c of row r in a 128-byte-row slice.
__device__ __forceinline__ int swz(int r, int c) { return r * kBK + ((c ^ (r & 7)) << 4); }

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

template <bool UP, int WM>
__global__ __launch_bounds__(Tile<WM>::kThreads) void mlp_kernel(MlpArgs a) {
    using TL = Tile<WM>;
    constexpr int kThreads = TL::kThreads, kBM = TL::kBM, kStageBytes = TL::kStageBytes, kStages = TL::kStages;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* stage = smem;                                  // [kStages][kStageBytes]
    const int KB = a.K / kBK;
    uint8_t* a_sc = smem + kStages * kStageBytes;           // [kBM][KB] E8M0
    uint8_t* w_sc = a_sc + kBM * KB;                        // [2][KB]
    int32_t* tot = (int32_t*)(smem + kStages * kStageBytes + ((kBM * KB + 2 * KB + 15) & ~15));
    int32_t* tpref = tot + a.E;                             // [E+1]

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1, g = lane >> 4, lr = lane & 15;

    // ---- which expert and row tile this block computes --------------------
    for (int e = tid; e < a.E; e += kThreads) {
        int st;
        tot[e] = (rows_of(a, e, st) + kBM - 1) / kBM;
    }
    __syncthreads();
    block_exclusive_scan<kThreads>(tot, tpref, a.E, 0);  // ends with a barrier
    const int slot = blockIdx.y;
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
    const int n0 = blockIdx.x * (UP ? kActN : kBR);

    // ---- scales of the whole K range, as E8M0 bytes ------------------------
    for (int i = tid; i < kBM * KB; i += kThreads) {
        const int r = i / KB, kb = i - r * KB;
        const int row = min(row0 + r, a.N - 1);
        a_sc[i] = (uint8_t)e8m0(a.as[(size_t)row * KB + kb]);
    }
    const int WRB = a.WR / kBK;
    for (int i = tid; i < 2 * KB; i += kThreads) {
        const int which = i / KB, kb = i - which * KB;
        int blk;
        if constexpr (UP) blk = (which == 0 ? n0 : a.I + n0) / kBK;
        else blk = min(n0 / kBK + which, WRB - 1);
        w_sc[i] = (uint8_t)e8m0(a.ws[((size_t)e * WRB + blk) * KB + kb]);
    }

    // ---- K loop -----------------------------------------------------------
    const uint8_t* wbase = a.w + (size_t)e * a.WR * a.K;
    // One slice (kBM rows of A and 256 weight rows, 128 bytes each) goes to
    // LDS by direct global->LDS copies: each instruction moves 1 KiB (8 rows)
    // with lane i filling LDS bytes [16i, 16i+16), so lane i fetches the
    // logical chunk that the swizzle puts at that position.
    const int pc = lane & 7, rl = lane >> 3;  // physical chunk, row within the 8-row group
    const int lc = pc ^ rl;                   // logical chunk held there
    auto issue = [&](int kb, int st) {
        uint8_t* sA = stage + st * kStageBytes;
#pragma unroll
        for (int j = 0; j < TL::kCopiesA; ++j) {
            const int q = TL::kCopiesA * w + j, r = 8 * q + rl;
            const int row = min(row0 + r, a.N - 1);
            __builtin_amdgcn_global_load_lds((const void*)(a.a + (size_t)row * a.K + kb * kBK + lc * 16),
                                             (__attribute__((address_space(3))) void*)(sA + q * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < TL::kCopiesB; ++j) {
            const int q = TL::kCopiesB * w + j, r = 8 * q + rl;
            __builtin_amdgcn_global_load_lds(
                (const void*)(wbase + (size_t)wrow_of<UP>(a, n0, r) * a.K + kb * kBK + lc * 16),
                (__attribute__((address_space(3))) void*)(sA + kBM * kBK + q * 1024), 16, 0, 0);
        }
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // 32 MFMAs of one 128-deep slice from LDS stage st
    auto compute = [&](int kb, int st) {
        const uint8_t* sA = stage + st * kStageBytes;
        const uint8_t* sB = sA + kBM * kBK;
        i32x8 af[4];
        int sa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 64 * wr + 16 * r + lr;
            const i32x4 lo4 = *(const i32x4*)(sA + swz(row, g));
            const i32x4 hi4 = *(const i32x4*)(sA + swz(row, g + 4));
            af[r] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            sa[r] = a_sc[row * KB + kb];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            int brow, sb;
            if constexpr (UP) {
                brow = (c < 4) ? 64 * wc + 16 * c : kActN + 64 * wc + 16 * (c - 4);
                sb = w_sc[(c < 4 ? 0 : 1) * KB + kb];
            } else {
                brow = 128 * wc + 16 * c;
                sb = w_sc[wc * KB + kb];
            }
            const int row = brow + lr;
            const i32x4 lo4 = *(const i32x4*)(sB + swz(row, g));
            const i32x4 hi4 = *(const i32x4*)(sB + swz(row, g + 4));
            const i32x8 bf = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[r], bf, acc[r][c], 0, 0, 0, sa[r],
                                                                             0, sb);
        }
    };

    // kStages-1 slices are in flight while one is multiplied.  Before each
    // barrier every wave waits until only its copies of the newer slices are
    // outstanding (s_waitcnt vmcnt counts them in issue order), so the barrier
    // publishes the next slice.  The barrier is the bare instruction: a
    // __syncthreads() release would also wait for the newest slice.  The
    // steady-state loop is unconditional so that nothing moves across its
    // wait; sched_barrier keeps the wait behind the slice's MFMAs.
    constexpr int kAhead = kStages - 1;
    constexpr int kLeft = (kAhead - 1) * TL::kCopies;  // copies allowed in flight at the barrier
    __syncthreads();  // scales in LDS
    for (int s = 0; s < kAhead; ++s)
        if (s < KB) issue(s, s);
    if (KB >= kAhead) wait_vm<kLeft>();
    else wait_vm<0>();
    bare_barrier();
    int kb = 0;
    for (; kb + kAhead < KB; ++kb) {
        issue(kb + kAhead, (kb + kAhead) % kStages);
        compute(kb, kb % kStages);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<kLeft>();
        bare_barrier();
    }
    for (; kb < KB; ++kb) {  // the last slices: nothing more to issue
        compute(kb, kb % kStages);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<0>();
        bare_barrier();
    }
    __syncthreads();

    if constexpr (UP) {
        // ---- SwiGLU, row amax over the tile's 128 act columns, FP8 codes -----
        // row strides padded by 16 bytes so the four rows a wave writes at
        // once (4 apart) fall in different LDS banks
        constexpr int kTS = kActN + 16;
        uint32_t* amx = (uint32_t*)stage;   // [2][kBM] |act| maxima of each wave column
        uint8_t* tile = stage + 4096;       // [kBM][kTS] codes
        float av[4][4][4];
        uint32_t rm[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t m = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float gg = acc[r][c][i], uu = acc[r][c + 4][i];
                    const float v = gg / (1.0f + exp_fixed(-gg)) * uu;
                    av[r][c][i] = v;
                    m = max(m, __float_as_uint(v) & 0x7FFFFFFFu);
                }
                rm[r][i] = row16_max_u32(m);
            }
        if (lr == 0)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) amx[wc * kBM + 64 * wr + 16 * r + 4 * g + i] = rm[r][i];
        __syncthreads();
        const int SI = a.I / kBK;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 64 * wr + 16 * r + 4 * g + i;
                const float amax = __uint_as_float(max(amx[row], amx[kBM + row]));
                const float aa = amax > 0x1p-100f ? amax : 0x1p-100f;
                float scale, inv;
                block_scale<true>(aa, scale, inv);
                const uint32_t q = pack_e4m3x4(av[r][0][i] * inv, av[r][1][i] * inv, av[r][2][i] * inv,
                                               av[r][3][i] * inv);
#pragma unroll
                for (int c = 0; c < 4; ++c) tile[row * kTS + 64 * wc + 16 * c + lr] = (uint8_t)(q >> (8 * c));
                if (wc == 0 && lr == 0 && row < nvalid) a.act_s[(size_t)(row0 + row) * SI + n0 / kBK] = scale;
            }
        __syncthreads();
        for (int i = tid; i < kBM * 8; i += kThreads) {
            const int r = i >> 3, c = i & 7;
            if (r < nvalid)
                *(u32x4*)(a.act + (size_t)(row0 + r) * a.I + n0 + c * 16) = *(const u32x4*)(tile + r * kTS + c * 16);
        }
    } else {
        // ---- BF16 output tile [kBM][256 + 8], staged for 16-byte stores ------
        // (rows padded by 16 bytes: the four rows a wave writes at once fall
        // in different LDS banks; the tile may run into the scale area, which
        // is no longer needed)
        constexpr int kTS = kBR + 8;
        uint16_t* tile = (uint16_t*)stage;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 64 * wr + 16 * r + 4 * g + i, col = 128 * wc + 16 * c + lr;
                    const __bf16 b = (__bf16)acc[r][c][i];
                    tile[row * kTS + col] = __builtin_bit_cast(uint16_t, b);
                }
        __syncthreads();
        for (int i = tid; i < kBM * 32; i += kThreads) {
            const int r = i >> 5, c = i & 31;
            const int col = n0 + c * 8;
            if (r < nvalid && col < a.WR)
                *(u32x4*)(a.y + (size_t)(row0 + r) * a.WR + col) = *(const u32x4*)(tile + r * kTS + c * 8);
        }
    }
}

// Dynamic LDS: the stages, the scales and the tile prefix; at least the
// epilogue's staging tile, which reuses the same bytes from the start.
template <int WM>
size_t lds_bytes_for(int K, int E) {
    using TL = Tile<WM>;
    const int KB = K / kBK;
    const size_t loop = TL::kStages * (size_t)TL::kStageBytes + (((size_t)TL::kBM * KB + 2 * KB + 15) & ~(size_t)15) +
                        4 * (2 * (size_t)E + 1);
    const size_t up_tile = 4096 + (size_t)TL::kBM * (kActN + 16);
    const size_t down_tile = (size_t)TL::kBM * (kBR + 8) * 2;
    return loop > up_tile ? (loop > down_tile ? loop : down_tile) : (up_tile > down_tile ? up_tile : down_tile);
}

// 256-row tiles when experts average at least 512 rows, else 128-row tiles.
int pick_wm(int N, int E) { return (long long)N >= 512LL * E ? 4 : 2; }

template <bool UP, int WM>
hipError_t launch_mlp(const MlpArgs& a, hipStream_t s) {
    const size_t lds = lds_bytes_for<WM>(a.K, a.E);
    const unsigned gx = UP ? (unsigned)(a.I / kActN) : (unsigned)((a.WR + kBR - 1) / kBR);
    const unsigned gy = (unsigned)(a.N / Tile<WM>::kBM + a.E);  // >= sum over experts of ceil(rows / BM)
    if (gx == 0 || gy == 0) return hipSuccess;
    hipLaunchKernelGGL((mlp_kernel<UP, WM>), dim3(gx, gy), dim3(Tile<WM>::kThreads), lds, s, a);
    return hipGetLastError();
}

template <bool UP>
hipError_t launch_pick(const MlpArgs& a, hipStream_t s) {
    return pick_wm(a.N, a.E) == 4 ? launch_mlp<UP, 4>(a, s) : launch_mlp<UP, 2>(a, s);
}

}  // namespace

size_t expert_mlp_lds_bytes(int N, int K, int E) {
    return pick_wm(N, E) == 4 ? lds_bytes_for<4>(K, E) : lds_bytes_for<2>(K, E);
}

// Raises the kernels' dynamic-LDS limit above the 64 KiB default (the
// attribute belongs to the function on the current device).
hipError_t prepare_expert_mlp(bool up, int N, int K, int E) {
    const int wm = pick_wm(N, E);
    const size_t lds = expert_mlp_lds_bytes(N, K, E);
    const void* f = up ? (wm == 4 ? (const void*)mlp_kernel<true, 4> : (const void*)mlp_kernel<true, 2>)
                       : (wm == 4 ? (const void*)mlp_kernel<false, 4> : (const void*)mlp_kernel<false, 2>);
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_expert_up(const int32_t* cnt_e, const int32_t* off_e, const uint8_t* x, const float* xs,
                            const uint8_t* w1, const float* w1s, uint8_t* act, float* act_s, int N, int H, int I,
                            int E, int C, hipStream_t stream) {
    MlpArgs a{};
    a.a = x;
    a.as = xs;
    a.w = w1;
    a.ws = w1s;
    a.cnt_e = cnt_e;
    a.off_e = off_e;
    a.act = act;
    a.act_s = act_s;
    a.N = N;
    a.K = H;
    a.WR = 2 * I;
    a.E = E;
    a.C = C;
    a.I = I;
    return launch_pick<true>(a, stream);
}

hipError_t launch_expert_down(const int32_t* cnt_e, const int32_t* off_e, const uint8_t* act, const float* act_s,
                              const uint8_t* w2, const float* w2s, uint16_t* y, int N, int H, int I, int E, int C,
                              hipStream_t stream) {
    MlpArgs a{};
    a.a = act;
    a.as = act_s;
    a.w = w2;
    a.ws = w2s;
    a.cnt_e = cnt_e;
    a.off_e = off_e;
    a.y = y;
    a.N = N;
    a.K = I;
    a.WR = H;
    a.E = E;
    a.C = C;
    a.I = I;
    return launch_pick<false>(a, stream);
}

}  // namespace cgl
