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
// passes run in a single launch with no workspace.  Batches of up to 32768
// tokens in the compact and padded layouts take a third design instead, one
// launch with one block per expert (layout_expert_kernel below); the
// two-pass kernels serve larger batches and the tile-aligned layout.
#include <mutex>
#include <type_traits>

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

// ---------------------------------------------------------------------------
// One-launch layout for batches of up to kExpertLayoutMaxTokens tokens in the
// compact and padded layouts, one block per expert.  Every block reads
// the whole routing table (at most 1 MiB, served by the L2 after the first
// block), so no workspace, no second launch and no count table are needed:
//   off_e[e] = #pairs with an index below e (compact and padded alike),
//   cnt_e[e] = #pairs routed to e,
//   rank of (t, j) in e's region = #tokens t' < t routed to e: token t is
//   thread t % 1024 of iteration t / 1024; each wave's 64-token ballot of
//   "routed to e" goes to LDS, an exclusive scan over (iteration, wave)
//   gives every ballot's base, and a popcount of the lanes below adds the
//   rest.
// Block e owns expert e; blocks of experts e < R also count cnt_r[e]
// (tokens with an expert on rank e).  Expert 0's block also checks every pair
// (an out-of-range or repeated index sets flag bit 1 and that pair's pos to
// -1) and, padded, counts every expert to raise bit 0; it writes the flags
// word.  (A separate checking block would be the 257th of a 256-CU chip and
// share a CU with an expert's block: measured slower, 11 against 7 us.)
// Expert e's block fills its own padded region's empty rows with -1, so no
// grid-wide fill precedes the positions.
// Per pair the expert blocks spend three compares (below e, equal to e, on
// rank e), unsigned so that out-of-range indices count nowhere.
// Blocks of NT threads: 1024 in general, 128 or 256 for batches that fit one
// iteration (fewer waves to launch and to meet at each barrier).
constexpr int kExpertLayoutThreads = 1024;
constexpr int kExpertLayoutMaxIters = 32;
constexpr int kExpertLayoutMaxTokens = kExpertLayoutThreads * kExpertLayoutMaxIters;
constexpr int kExpertLayoutBatch = 4;  // iterations whose loads are in flight together

// Inclusive scan over the wave: DPP row_shr inside rows of 16 (lanes without
// a source read 0), then the row totals added on.
__device__ __forceinline__ int wave_scan_dpp(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

template <int KT, int NT>
__global__ __launch_bounds__(NT) void layout_expert_kernel(LayoutArgs a) {
    constexpr int kWaves = NT / kWave, kMaxIters = kExpertLayoutMaxTokens / NT;
    __shared__ uint64_t ballots[kMaxIters * kWaves];
    __shared__ int32_t base[kMaxIters * kWaves];
    __shared__ int8_t slot[kExpertLayoutMaxTokens];  // slot of e in the token, or -1
    __shared__ int32_t hist[512];                    // expert 0, padded: counts
    __shared__ int32_t red[2][kWaves];
    __shared__ int32_t total;
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = a.T, k = KT > 0 ? KT : a.k;
    const int iters = (T + NT - 1) / NT;
    const int Er = a.E / a.R;
    const bool rank_block = e < a.R;
    const unsigned r0 = (unsigned)(e * Er);  // first expert of rank e (rank blocks)
    const bool check = e == 0;               // block-uniform
    const bool count_all = check && a.C > 0;
    if (count_all) {
        for (int i = tid; i < a.E; i += NT) hist[i] = 0;
        __syncthreads();
    }

    int lt = 0, rk = 0, bad = 0;
    // The walk over the tokens, compiled twice: with the pair check for expert
    // 0's block and without it for the others.  One copy with a runtime check
    // slowed every block: 10.0 us per launch at 4096 tokens top-8 of 256,
    // against 7.8 us for the two copies (6.7 us with no check at all; the
    // check in a second walk of its own, 10.3 us).
    const auto walk = [&](auto check_tag) {
        constexpr bool CHECK = decltype(check_tag)::value;
        for (int it0 = 0; it0 < iters; it0 += kExpertLayoutBatch) {
            TokenRow<KT> rows[kExpertLayoutBatch];
#pragma unroll
            for (int b = 0; b < kExpertLayoutBatch; ++b) {
                const int t = (it0 + b) * NT + tid;
                if (KT > 0 && it0 + b < iters && t < T) rows[b].load(a.idx + (size_t)t * k);
            }
#pragma unroll
            for (int b = 0; b < kExpertLayoutBatch; ++b) {
                const int it = it0 + b;
                if (it >= iters) break;  // block-uniform
                const int t = it * NT + tid;
                int js = -1;
                if (t < T) {
                    bool hit_rank = false;
                    // slots in descending order, so js ends as the first slot
                    // holding e (a repeated index is flagged by expert 0's block)
                    for (int j = (KT > 0 ? KT : k) - 1; j >= 0; --j) {
                        const unsigned ej = (unsigned)(KT > 0 ? rows[b].e[j] : a.idx[(size_t)t * k + j]);
                        lt += ej < (unsigned)e ? 1 : 0;
                        js = ej == (unsigned)e ? j : js;
                        hit_rank |= ej - r0 < (unsigned)Er;
                    }
                    rk += (rank_block && hit_rank) ? 1 : 0;
                    if constexpr (CHECK) {
                        // every pair: an index outside [0, E) or repeated in the
                        // token raises the flag (branch-free; the pairs' pos -1
                        // is written only in waves that saw one); padded, the
                        // counts of every expert for the overflow flag
                        const auto bad_pair = [&](int j) {
                            const int ej = KT > 0 ? rows[b].e[j] : a.idx[(size_t)t * k + j];
                            bool dup = false;
                            for (int i = 0; i < j; ++i) dup |= (KT > 0 ? rows[b].e[i] : a.idx[(size_t)t * k + i]) == ej;
                            return (unsigned)ej >= (unsigned)a.E || dup;
                        };
                        bool tbad = false;
                        for (int j = 0; j < (KT > 0 ? KT : k); ++j) tbad |= bad_pair(j);
                        bad |= tbad ? 1 : 0;
                        if (__ballot(tbad)) {  // rare
                            for (int j = 0; j < (KT > 0 ? KT : k); ++j)
                                if (tbad && bad_pair(j)) a.pos[(size_t)t * k + j] = -1;
                        }
                        if (count_all)
                            for (int j = 0; j < (KT > 0 ? KT : k); ++j)
                                if (!bad_pair(j)) atomicAdd(&hist[KT > 0 ? rows[b].e[j] : a.idx[(size_t)t * k + j]], 1);
                    }
                }
                slot[it * NT + tid] = (int8_t)js;
                const uint64_t bal = __ballot(js >= 0);
                if (lane == 0) ballots[it * kWaves + w] = bal;
            }
        }
    };
    if (check)
        walk(std::true_type{});
    else
        walk(std::false_type{});
    if (check) {
        int over = 0;
        if (count_all) {
            __syncthreads();  // every pair counted
            for (int i = tid; i < a.E; i += NT) over |= hist[i] > a.C;
        }
        const int any_over = __syncthreads_or(over);
        const int any_bad = __syncthreads_or(bad);
        if (tid == 0) a.flags[0] = (any_over ? 1 : 0) | (any_bad ? 2 : 0);
    }
    // block sums of lt and rk
    const int s0 = wave_sum(lt), s1 = wave_sum(rk);
    if (lane == 0) {
        red[0][w] = s0;
        red[1][w] = s1;
    }
    __syncthreads();
    // exclusive scan of the ballots' popcounts over (iteration, wave), by wave 0
    const int nb = iters * kWaves;
    if (w == 0) {
        int carry = 0;
        for (int i0 = 0; i0 < nb; i0 += kWave) {
            const int i = i0 + lane;
            const int c = i < nb ? __popcll(ballots[i]) : 0;
            const int inc = wave_scan_dpp(c);
            if (i < nb) base[i] = carry + inc - c;
            carry += __builtin_amdgcn_readlane(inc, 63);
        }
        if (lane == 0) total = carry;
    }
    __syncthreads();
    int off = 0, cr = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
        off += red[0][q];
        cr += red[1][q];
    }
    const int cnt = total;

    // positions and receive rows of expert e's pairs
    const uint64_t below = (1ull << lane) - 1ull;
    for (int it = 0; it < iters; ++it) {
        const int js = slot[it * NT + tid];
        if (js < 0) continue;
        const int t = it * NT + tid;
        const int i = it * kWaves + w;
        const int rank = base[i] + __popcll(ballots[i] & below);
        int p;
        if (a.C == 0)
            p = off + rank;
        else
            p = rank < a.C ? e * a.C + rank : -1;
        a.pos[(size_t)t * k + js] = p;
        if (p >= 0) a.recv_src[p] = t * k + js;
    }
    // padded: this expert's empty rows
    if (a.C > 0)
        for (int r = min(cnt, a.C) + tid; r < a.C; r += NT) a.recv_src[(size_t)e * a.C + r] = -1;

    // counts and offsets
    if (tid == 0) {
        a.cnt_e[e] = cnt;
        a.off_e[e] = off;
        if (e == a.E - 1) a.off_e[a.E] = off + cnt;
        if (rank_block) a.cnt_r[e] = cr;
        if (e % Er == 0) a.off_r[e / Er] = off;
        if (e == a.E - 1) a.off_r[a.R] = off + cnt;
    }
}

size_t lds_bytes(int E, int R, bool with_table) {
    return sizeof(uint64_t) * (size_t)kLayoutWaves * (E + R) + (with_table ? sizeof(int32_t) * kTableCacheInts : 0) +
           sizeof(int32_t) * (3 * (size_t)E + 1);
}

// The per-expert kernel's time grows with the batch (every block walks all of
// it) and hardly with E; the two-pass kernels split the batch over blocks.
// Measured back to back: 4096 tokens top-8, E 8..256: 9.2-9.6 us against
// 11.1-12.6 us; 16384 tokens top-2: E <= 64 10.9-11.4 us against 9.7-10.3 us,
// E 128 and 256 10.7-10.9 us against 17.4-18.0 us.
inline bool use_expert_layout(const LayoutArgs& a) {
    return a.A <= 1 && a.T > 0 && a.T <= kExpertLayoutMaxTokens && (a.T <= 8192 || a.E > 64);
}

template <int KT>
hipError_t launch_kt(LayoutArgs a, hipStream_t stream) {
    if (use_expert_layout(a)) {
        if (a.T <= 128)
            hipLaunchKernelGGL((layout_expert_kernel<KT, 128>), dim3(a.E), dim3(128), 0, stream, a);
        else if (a.T <= 256)
            hipLaunchKernelGGL((layout_expert_kernel<KT, 256>), dim3(a.E), dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((layout_expert_kernel<KT, kExpertLayoutThreads>), dim3(a.E),
                               dim3(kExpertLayoutThreads), 0, stream, a);
        return hipGetLastError();
    }
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
