// layout.hip -- routing layout: a stable counting sort of the (token, slot)
// pairs by expert, with no global atomics.
//
// Follows "Efficient and Portable Mixture-of-Experts Communication"
// (Perplexity), sections "Portable kernels" (fixed per-expert capacity gives
// every sender a unique destination address without coordination) and
// "Dispatch" (per-expert counts; source token index kept for the combine),
// and the DeepEP V2 digest, section "training/prefill/decoding usage"
// (per-expert token counts for the grouped GEMM).
//
// Tokens are cut into blocks of 256 (four waves of 64, one token per lane).
// Each wave builds one 64-bit lane mask per expert (and per rank) in LDS with
// ds_or_b64; popcounts give the per-block counts, and a pair's rank among the
// earlier pairs of its expert is
//     (pairs in earlier blocks) + (pairs in earlier waves of this block)
//     + popcount(its wave's mask & lanes below it).
// Pass 1 writes per-block count rows to the workspace.  Pass 2 pulls the
// whole count table into LDS in one cooperative sweep, so every block gets
// its prefix, the totals and the exclusive scan over experts without another
// launch, then writes pos / recv_src.  When one block covers all tokens both
// passes run in a single launch with no workspace.
#include <mutex>

#include "moe_device.hpp"
#include "moe_internal.hpp"

// The count table of moe_get_layout_noalloc: a library-owned copy of the
// layout workspace, one per GPU, held until the process ends.  Host code never
// passes this name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[cgl::kLayoutScratchBytes];

namespace cgl {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kTokensPerLayoutBlock = kLayoutThreads;  // one token per thread
constexpr int kTableCacheInts = 8192;                  // count rows kept in LDS (32 KiB)

struct LayoutArgs {
    const int32_t* idx;
    int32_t *cnt_e, *cnt_r, *off_e, *off_r, *pos, *recv_src, *flags;
    int32_t* ws_cnt;    // [NB, E] per-block expert counts
    int32_t* ws_rcnt;   // [NB, R] per-block distinct-token rank counts
    int32_t* ws_bad;    // [NB]    per-block bad-index flag
    int T, E, k, R, C, A, NB;  // A > 1: expert regions start on multiples of A rows
    int tab_ints;       // LDS ints reserved for the cached count table (0: none)
};

// A token's k expert indices, loaded with 16/8-byte vector loads when k is a
// compile-time 8, 4 or 2 (KT); KT = 0 handles any k up to 64 in a loop.
template <int KT>
struct TokenRow {
    static constexpr int N = KT > 0 ? KT : 1;
    int e[N];
    __device__ __forceinline__ void load(const int32_t* row) {
        if constexpr (KT % 4 == 0) {
#pragma unroll
            for (int q = 0; q < KT; q += 4) {
                const int4 v = *(const int4*)(row + q);
                e[q] = v.x; e[q + 1] = v.y; e[q + 2] = v.z; e[q + 3] = v.w;
            }
        } else if constexpr (KT == 2) {
            const int2 v = *(const int2*)row;
            e[0] = v.x; e[1] = v.y;
        } else if constexpr (KT > 0) {
#pragma unroll
            for (int q = 0; q < KT; ++q) e[q] = row[q];
        }
    }
};

// Builds the lane masks of this block's tokens.  Returns 1 in any thread that
// saw an index outside [0, E) or an index repeated inside its token.
template <int KT>
__device__ int build_masks(const LayoutArgs& a, uint64_t* emask, uint64_t* rmask, const TokenRow<KT>& tr,
                           bool have) {
    const int tid = threadIdx.x;
    for (int i = tid; i < kLayoutWaves * a.E; i += kLayoutThreads) emask[i] = 0;
    for (int i = tid; i < kLayoutWaves * a.R; i += kLayoutThreads) rmask[i] = 0;
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63;
    const int Er = a.E / a.R;
    const uint64_t bit = 1ull << lane;
    int bad = 0;
    if (have) {
        const int t = blockIdx.x * kTokensPerLayoutBlock + tid;
        const int kk = KT > 0 ? KT : a.k;
#pragma unroll
        for (int j = 0; j < (KT > 0 ? KT : 64); ++j) {
            if (KT == 0 && j >= kk) break;
            const int e = KT > 0 ? tr.e[j] : a.idx[(size_t)t * a.k + j];
            if (e < 0 || e >= a.E) {
                bad = 1;
                continue;
            }
            const uint64_t old = atomicOr((unsigned long long*)&emask[w * a.E + e], (unsigned long long)bit);
            if (old & bit) bad = 1;
            atomicOr((unsigned long long*)&rmask[w * a.R + e / Er], (unsigned long long)bit);
        }
    }
    __syncthreads();
    return bad;
}

// recv_src[i] = -1 for i in [0, n), cooperatively by `nthreads` threads with
// index `tid` (16-byte stores when the array is 16-byte aligned).
__device__ void fill_minus_one(int32_t* recv_src, size_t n, size_t tid, size_t nthreads) {
    if (((uintptr_t)recv_src & 15) == 0) {
        const int4 m = make_int4(-1, -1, -1, -1);
        for (size_t i = tid; i < n / 4; i += nthreads) ((int4*)recv_src)[i] = m;
        for (size_t i = (n / 4) * 4 + tid; i < n; i += nthreads) recv_src[i] = -1;
    } else {
        for (size_t i = tid; i < n; i += nthreads) recv_src[i] = -1;
    }
}

__device__ __forceinline__ size_t recv_rows(const LayoutArgs& a) {
    return a.C > 0 ? (size_t)a.E * a.C : (size_t)a.T * a.k + (a.A > 1 ? (size_t)a.E * (a.A - 1) : 0);
}

__device__ __forceinline__ int block_count(const uint64_t* mask, int stride, int i) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) c += __popcll(mask[w * stride + i]);
    return c;
}

// Pass 1: per-block count rows.
template <int KT>
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(LayoutArgs a) {
    extern __shared__ uint64_t lds[];
    uint64_t* emask = lds;
    uint64_t* rmask = lds + kLayoutWaves * a.E;
    const int t = blockIdx.x * kTokensPerLayoutBlock + threadIdx.x;
    const bool have = t < a.T;
    TokenRow<KT> tr;
    if (have) tr.load(a.idx + (size_t)t * a.k);
    // padded and aligned modes: every receive row starts empty; pass 2 (a
    // later launch) writes the occupied ones
    if (a.C > 0 || a.A > 1)
        fill_minus_one(a.recv_src, recv_rows(a), (size_t)blockIdx.x * kLayoutThreads + threadIdx.x,
                       (size_t)gridDim.x * kLayoutThreads);
    const int bad = build_masks<KT>(a, emask, rmask, tr, have);
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < a.E; e += kLayoutThreads) a.ws_cnt[(size_t)b * a.E + e] = block_count(emask, a.E, e);
    for (int r = threadIdx.x; r < a.R; r += kLayoutThreads)
        a.ws_rcnt[(size_t)b * a.R + r] = block_count(rmask, a.R, r);
    const int any_bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) a.ws_bad[b] = any_bad;
}

// Pass 2 (FUSED: the only block, counts taken from its own masks).
template <int KT, bool FUSED>
__global__ __launch_bounds__(kLayoutThreads) void layout_position_kernel(LayoutArgs a) {
    extern __shared__ uint64_t lds[];
    uint64_t* emask = lds;
    uint64_t* rmask = lds + kLayoutWaves * a.E;
    int32_t* tab = (int32_t*)(rmask + kLayoutWaves * a.R);  // cached count rows (16-byte aligned)
    int32_t* pre = tab + a.tab_ints;                         // [E] pairs in earlier blocks
    int32_t* tot = pre + a.E;                                // [E] totals
    int32_t* off = tot + a.E;                                // [E+1] exclusive scan

    const int b = blockIdx.x, tid = threadIdx.x;
    const int t = b * kTokensPerLayoutBlock + tid;
    const bool have = t < a.T;
    TokenRow<KT> tr;
    if (have) tr.load(a.idx + (size_t)t * a.k);

    // ---- pull the count tables (all blocks' rows) into LDS -----------------
    // [NB*E] expert counts, then [NB*R] rank counts, then [NB] bad flags: one
    // cooperative sweep of independent loads, issued before any is used.
    const int nE = a.NB * a.E, nR = a.NB * a.R;
    const bool cached = !FUSED && nE + nR + a.NB <= a.tab_ints;
    if (cached) {
        const int n = nE + nR + a.NB;  // the three arrays are contiguous in the workspace
        if ((n & 3) == 0) {
            const int4* src = (const int4*)a.ws_cnt;
            int4* dst = (int4*)tab;
            for (int i = tid; i < n / 4; i += kLayoutThreads) dst[i] = src[i];
        } else {
            for (int i = tid; i < n; i += kLayoutThreads) tab[i] = a.ws_cnt[i];
        }
    }
    // padded and aligned modes, single block: empty every receive row before
    // the barrier in build_masks; the positions below overwrite the occupied ones
    if (FUSED && (a.C > 0 || a.A > 1)) fill_minus_one(a.recv_src, recv_rows(a), tid, kLayoutThreads);
    const int bad_here = build_masks<KT>(a, emask, rmask, tr, have);  // contains __syncthreads

    // ---- block prefix and totals per expert -------------------------------
    for (int e = tid; e < a.E; e += kLayoutThreads) {
        if (FUSED) {
            pre[e] = 0;
            tot[e] = block_count(emask, a.E, e);
        } else {
            int p = 0, s = 0;
            if (cached) {
                for (int bb = 0; bb < a.NB; ++bb) {
                    const int c = tab[bb * a.E + e];
                    p += (bb < b) ? c : 0;
                    s += c;
                }
            } else {
                int bb = 0;
                for (; bb + 8 <= a.NB; bb += 8) {
                    int c[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) c[q] = a.ws_cnt[(size_t)(bb + q) * a.E + e];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        p += (bb + q < b) ? c[q] : 0;
                        s += c[q];
                    }
                }
                for (; bb < a.NB; ++bb) {
                    const int c = a.ws_cnt[(size_t)bb * a.E + e];
                    p += (bb < b) ? c : 0;
                    s += c;
                }
            }
            pre[e] = p;
            tot[e] = s;
        }
    }
    __syncthreads();
    block_exclusive_scan<kLayoutThreads>(tot, off, a.E, a.A);

    // ---- block 0 publishes counts, offsets and flags ----------------------
    if (b == 0) {
        const int Er = a.E / a.R;
        for (int e = tid; e < a.E; e += kLayoutThreads) a.cnt_e[e] = tot[e];
        for (int e = tid; e <= a.E; e += kLayoutThreads) a.off_e[e] = off[e];
        for (int r = tid; r < a.R; r += kLayoutThreads) {
            int c = 0;
            if (FUSED) {
                c = block_count(rmask, a.R, r);
            } else if (cached) {
                for (int bb = 0; bb < a.NB; ++bb) c += tab[nE + bb * a.R + r];
            } else {
                for (int bb = 0; bb < a.NB; ++bb) c += a.ws_rcnt[(size_t)bb * a.R + r];
            }
            a.cnt_r[r] = c;
        }
        for (int r = tid; r <= a.R; r += kLayoutThreads) a.off_r[r] = off[r * Er];
        int f = 0;
        if (a.C > 0)
            for (int e = tid; e < a.E; e += kLayoutThreads)
                if (tot[e] > a.C) f |= 1;
        if (FUSED) {
            if (bad_here) f |= 2;
        } else {
            for (int bb = tid; bb < a.NB; bb += kLayoutThreads)
                if (cached ? tab[nE + nR + bb] : a.ws_bad[bb]) f |= 2;
        }
        const int any_over = __syncthreads_or(f & 1);
        const int any_bad = __syncthreads_or(f & 2);
        if (tid == 0) a.flags[0] = (any_over ? 1 : 0) | (any_bad ? 2 : 0);
    }

    // ---- positions ----------------------------------------------------------
    const int w = tid >> 6, lane = tid & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    if (have) {
        const int kk = KT > 0 ? KT : a.k;
        int32_t* prow = a.pos + (size_t)t * a.k;
        int pv[KT > 0 ? KT : 1];
#pragma unroll
        for (int j = 0; j < (KT > 0 ? KT : 64); ++j) {
            if (KT == 0 && j >= kk) break;
            const int e = KT > 0 ? tr.e[j] : a.idx[(size_t)t * a.k + j];
            int32_t p = -1;
            if (e >= 0 && e < a.E) {
                int rank = pre[e] + __popcll(emask[w * a.E + e] & below);
#pragma unroll
                for (int ww = 0; ww < kLayoutWaves - 1; ++ww)
                    if (ww < w) rank += __popcll(emask[ww * a.E + e]);
                if (a.C == 0)
                    p = off[e] + rank;
                else if (rank < a.C)
                    p = e * a.C + rank;
            }
            if (p >= 0) a.recv_src[p] = t * a.k + j;
            if constexpr (KT > 0)
                pv[j] = p;
            else
                prow[j] = p;
        }
        if constexpr (KT % 4 == 0 && KT > 0) {
#pragma unroll
            for (int q = 0; q < KT; q += 4) *(int4*)(prow + q) = make_int4(pv[q], pv[q + 1], pv[q + 2], pv[q + 3]);
        } else if constexpr (KT == 2) {
            *(int2*)prow = make_int2(pv[0], pv[1]);
        } else if constexpr (KT > 0) {
#pragma unroll
            for (int q = 0; q < KT; ++q) prow[q] = pv[q];
        }
    }

}

size_t lds_bytes(int E, int R, bool with_table) {
    return sizeof(uint64_t) * (size_t)kLayoutWaves * (E + R) + (with_table ? sizeof(int32_t) * kTableCacheInts : 0) +
           sizeof(int32_t) * (3 * (size_t)E + 1);
}

template <int KT>
hipError_t launch_kt(LayoutArgs a, hipStream_t stream) {
    if (a.NB <= 1) {
        a.tab_ints = 0;
        hipLaunchKernelGGL((layout_position_kernel<KT, true>), dim3(1), dim3(kLayoutThreads),
                           lds_bytes(a.E, a.R, false), stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((layout_count_kernel<KT>), dim3(a.NB), dim3(kLayoutThreads),
                       sizeof(uint64_t) * (size_t)kLayoutWaves * (a.E + a.R), stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bool table = a.NB * (a.E + a.R + 1) <= kTableCacheInts;
    a.tab_ints = table ? kTableCacheInts : 0;
    hipLaunchKernelGGL((layout_position_kernel<KT, false>), dim3(a.NB), dim3(kLayoutThreads),
                       lds_bytes(a.E, a.R, table), stream, a);
    return hipGetLastError();
}

}  // namespace

size_t layout_workspace_bytes(int T, int E, int R) {
    const int NB = (T + kTokensPerLayoutBlock - 1) / kTokensPerLayoutBlock;
    return sizeof(int32_t) * ((size_t)NB * (E + R + 1)) + 256;
}

hipError_t launch_layout(const int32_t* idx, int32_t* cnt_e, int32_t* cnt_r, int32_t* off_e, int32_t* off_r,
                         int32_t* pos, int32_t* recv_src, int32_t* flags, void* workspace, int T, int E, int k,
                         int R, int C, int A, hipStream_t stream) {
    const int NB = (T + kTokensPerLayoutBlock - 1) / kTokensPerLayoutBlock;
    LayoutArgs a{};
    a.idx = idx;
    a.cnt_e = cnt_e;
    a.cnt_r = cnt_r;
    a.off_e = off_e;
    a.off_r = off_r;
    a.pos = pos;
    a.recv_src = recv_src;
    a.flags = flags;
    a.T = T;
    a.E = E;
    a.k = k;
    a.R = R;
    a.C = C;
    a.A = A;
    a.NB = NB > 0 ? NB : 1;
    int32_t* ws = (int32_t*)workspace;
    a.ws_cnt = ws;
    a.ws_rcnt = ws + (size_t)a.NB * E;
    a.ws_bad = ws + (size_t)a.NB * (E + R);
    // vector paths need 16-byte aligned rows (k = 8, 4) or 8-byte (k = 2)
    const bool al16 = ((uintptr_t)idx % 16 == 0) && ((uintptr_t)pos % 16 == 0);
    const bool al8 = ((uintptr_t)idx % 8 == 0) && ((uintptr_t)pos % 8 == 0);
    if (k == 8 && al16) return launch_kt<8>(a, stream);
    if (k == 4 && al16) return launch_kt<4>(a, stream);
    if (k == 2 && al8) return launch_kt<2>(a, stream);
    return launch_kt<0>(a, stream);
}

size_t layout_lds_bytes_host(int E, int R) { return lds_bytes(E, R, true); }

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device ordinal
}  // namespace

hipError_t layout_scratch(void** ptr) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // first call on this device, which is current: look the symbol up once
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace cgl
