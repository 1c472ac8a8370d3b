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
// Tokens are cut into blocks of 256 (four waves of 64).  In a block, each
// wave builds one 64-bit lane mask per expert (and per rank) in LDS with
// ds_or_b64; popcounts give the per-block counts, and a token's rank among
// the earlier tokens of its expert is
//     (pairs in earlier blocks) + (pairs in earlier waves of this block)
//     + popcount(mask of its wave & lanes below it).
// Pass 1 writes per-block count rows to the workspace; pass 2 lets every
// block sum the rows before it (and all rows, for the totals and the
// exclusive scan over experts) and then writes pos / recv_src.  When a single
// block covers all tokens both passes run in one launch with no workspace.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kTokensPerLayoutBlock = kLayoutThreads;  // one token per thread

struct LayoutArgs {
    const int32_t* idx;
    int32_t *cnt_e, *cnt_r, *off_e, *off_r, *pos, *recv_src, *flags;
    int32_t* ws_cnt;    // [NB, E] per-block expert counts
    int32_t* ws_rcnt;   // [NB, R] per-block distinct-token rank counts
    int32_t* ws_bad;    // [NB]    per-block bad-index flag
    int T, E, k, R, C, NB;
};

// LDS: emask[kLayoutWaves][E], rmask[kLayoutWaves][R] (u64), then int32
// scratch of 3*E + 1 words (block prefix, totals, exclusive offsets).
__host__ __device__ inline size_t layout_lds_bytes(int E, int R) {
    return sizeof(uint64_t) * (size_t)kLayoutWaves * (E + R) + sizeof(int32_t) * (3 * (size_t)E + 1);
}

// Builds the masks of this block's tokens; returns 1 in any thread that saw a
// bad index.
__device__ int build_masks(const LayoutArgs& a, uint64_t* emask, uint64_t* rmask) {
    const int tid = threadIdx.x;
    for (int i = tid; i < kLayoutWaves * a.E; i += kLayoutThreads) emask[i] = 0;
    for (int i = tid; i < kLayoutWaves * a.R; i += kLayoutThreads) rmask[i] = 0;
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63;
    const int t = blockIdx.x * kTokensPerLayoutBlock + tid;
    const int Er = a.E / a.R;
    const uint64_t bit = 1ull << lane;
    int bad = 0;
    if (t < a.T) {
        const int32_t* row = a.idx + (size_t)t * a.k;
        for (int j = 0; j < a.k; ++j) {
            const int e = row[j];
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

__device__ __forceinline__ int block_count(const uint64_t* mask, int stride, int i) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) c += __popcll(mask[w * stride + i]);
    return c;
}

// Pass 1: per-block count rows.
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(LayoutArgs a) {
    extern __shared__ uint64_t lds[];
    uint64_t* emask = lds;
    uint64_t* rmask = lds + kLayoutWaves * a.E;
    const int bad = build_masks(a, emask, rmask);
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < a.E; e += kLayoutThreads)
        a.ws_cnt[(size_t)b * a.E + e] = block_count(emask, a.E, e);
    for (int r = threadIdx.x; r < a.R; r += kLayoutThreads)
        a.ws_rcnt[(size_t)b * a.R + r] = block_count(rmask, a.R, r);
    const int any_bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) a.ws_bad[b] = any_bad;
}

// Exclusive scan of tot[0..E) into off[0..E] (off[E] = total), block-wide.
__device__ void block_exclusive_scan(const int32_t* tot, int32_t* off, int E) {
    // each thread scans a contiguous run of experts; then a scan of the run sums
    __shared__ int32_t part[kLayoutThreads];
    const int tid = threadIdx.x;
    const int per = (E + kLayoutThreads - 1) / kLayoutThreads;
    const int lo = min(tid * per, E), hi = min(lo + per, E);
    int s = 0;
    for (int e = lo; e < hi; ++e) s += tot[e];
    part[tid] = s;
    __syncthreads();
    // Hillis-Steele over 256 partial sums
    for (int d = 1; d < kLayoutThreads; d <<= 1) {
        const int v = (tid >= d) ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = (tid == 0) ? 0 : part[tid - 1];
    for (int e = lo; e < hi; ++e) {
        off[e] = run;
        run += tot[e];
    }
    if (tid == kLayoutThreads - 1) off[E] = part[kLayoutThreads - 1];
    __syncthreads();
}

// Pass 2 (FUSED: the only block, counts taken from its own masks).
template <bool FUSED>
__global__ __launch_bounds__(kLayoutThreads) void layout_position_kernel(LayoutArgs a) {
    extern __shared__ uint64_t lds[];
    uint64_t* emask = lds;
    uint64_t* rmask = lds + kLayoutWaves * a.E;
    int32_t* pre = (int32_t*)(rmask + kLayoutWaves * a.R);  // [E] pairs in earlier blocks
    int32_t* tot = pre + a.E;                                // [E] totals
    int32_t* off = tot + a.E;                                // [E+1] exclusive scan

    const int b = blockIdx.x, tid = threadIdx.x;
    const int bad_here = build_masks(a, emask, rmask);

    // ---- block prefix and totals per expert ------------------------------
    for (int e = tid; e < a.E; e += kLayoutThreads) {
        if (FUSED) {
            pre[e] = 0;
            tot[e] = block_count(emask, a.E, e);
        } else {
            int p = 0, s = 0;
            for (int bb = 0; bb < a.NB; ++bb) {
                const int c = a.ws_cnt[(size_t)bb * a.E + e];
                if (bb < b) p += c;
                s += c;
            }
            pre[e] = p;
            tot[e] = s;
        }
    }
    __syncthreads();
    block_exclusive_scan(tot, off, a.E);

    // ---- block 0 publishes counts, offsets and flags ----------------------
    if (b == 0) {
        const int Er = a.E / a.R;
        for (int e = tid; e < a.E; e += kLayoutThreads) a.cnt_e[e] = tot[e];
        for (int e = tid; e <= a.E; e += kLayoutThreads) a.off_e[e] = off[e];
        for (int r = tid; r < a.R; r += kLayoutThreads) {
            int c = 0;
            if (FUSED) {
                c = block_count(rmask, a.R, r);
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
                if (a.ws_bad[bb]) f |= 2;
        }
        const int any_over = __syncthreads_or(f & 1);
        const int any_bad = __syncthreads_or(f & 2);
        if (tid == 0) a.flags[0] = (any_over ? 1 : 0) | (any_bad ? 2 : 0);
    }

    // ---- positions --------------------------------------------------------
    const int w = tid >> 6, lane = tid & 63;
    const int t = b * kTokensPerLayoutBlock + tid;
    const uint64_t below = (1ull << lane) - 1ull;
    if (t < a.T) {
        const int32_t* row = a.idx + (size_t)t * a.k;
        for (int j = 0; j < a.k; ++j) {
            const int e = row[j];
            int32_t p = -1;
            if (e >= 0 && e < a.E) {
                int rank = pre[e] + __popcll(emask[w * a.E + e] & below);
                for (int ww = 0; ww < w; ++ww) rank += __popcll(emask[ww * a.E + e]);
                if (a.C == 0)
                    p = off[e] + rank;
                else if (rank < a.C)
                    p = e * a.C + rank;
            }
            a.pos[(size_t)t * a.k + j] = p;
            if (p >= 0) a.recv_src[p] = t * a.k + j;
        }
    }

    // ---- padded mode: mark the empty rows of experts e = b, b+NB, ... -----
    if (a.C > 0) {
        for (int e = b; e < a.E; e += a.NB) {
            const int used = min(tot[e], a.C);
            for (int r = used + tid; r < a.C; r += kLayoutThreads) a.recv_src[(size_t)e * a.C + r] = -1;
        }
    }
}

}  // namespace

size_t layout_workspace_bytes(int T, int E, int R) {
    const int NB = (T + kTokensPerLayoutBlock - 1) / kTokensPerLayoutBlock;
    return sizeof(int32_t) * ((size_t)NB * (E + R + 1)) + 256;
}

hipError_t launch_layout(const int32_t* idx, int32_t* cnt_e, int32_t* cnt_r, int32_t* off_e, int32_t* off_r,
                         int32_t* pos, int32_t* recv_src, int32_t* flags, void* workspace, int T, int E,
                         int k, int R, int C, hipStream_t stream) {
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
    a.NB = NB > 0 ? NB : 1;
    const size_t lds = layout_lds_bytes(E, R);
    if (NB <= 1) {
        hipLaunchKernelGGL((layout_position_kernel<true>), dim3(1), dim3(kLayoutThreads), lds, stream, a);
        return hipGetLastError();
    }
    int32_t* ws = (int32_t*)workspace;
    a.ws_cnt = ws;
    a.ws_rcnt = ws + (size_t)NB * E;
    a.ws_bad = ws + (size_t)NB * (E + R);
    hipLaunchKernelGGL(layout_count_kernel, dim3(NB), dim3(kLayoutThreads),
                       sizeof(uint64_t) * (size_t)kLayoutWaves * (E + R), stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((layout_position_kernel<false>), dim3(NB), dim3(kLayoutThreads), lds, stream, a);
    return hipGetLastError();
}

size_t layout_lds_bytes_host(int E, int R) { return layout_lds_bytes(E, R); }

}  // namespace cgl
