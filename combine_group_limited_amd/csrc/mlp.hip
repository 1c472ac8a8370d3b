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
// one per 128x128 block -- so each 64-deep step is one
// v_mfma_scale_f32_32x32x64_f8f6f4 per 32x32 output tile with both scales
// handed to the instruction as E8M0 exponents: no rescaling on the vector
// units.  Instruction facts used (measured on gfx950): lane l supplies row
// l%32 of each operand and one half of the 64-deep K range (which bytes does
// not matter as long as both operands agree, since a 128-deep scale block
// covers the whole step); lane l also supplies the scale of row l%32, and the
// op_sel field picks which byte of the 32-bit scale register is used, so the
// scales of four row tiles travel in one register; accumulator element i of
// lane l is row 8(i/4) + 4(l/32) + i%4, column l%32.
//
// Tiles: a block of four waves (2 x 2) owns BM = 64*TM rows of one expert x
// 256 weight rows; wave (wr, wc) owns 32*TM rows x 128 weight rows = TM x 4
// MFMA tiles (TM = 4: 256 accumulators per lane, one wave per SIMD).  Up:
// the block's weight rows are 128 gate rows and the matching 128 up rows, and
// wave wc takes gate rows 64wc.. and the same up rows, so SwiGLU pairs
// registers of one lane; down: 256 output columns.  The K loop moves
// 128-deep stages of both operands (whole 128-byte lines per row) through
// two LDS buffers (three for 128-row tiles) filled by direct global->LDS
// copies; 16-byte chunks are XOR-swizzled by row so fragment reads are
// conflict-free.  Each stage is computed as two 64-deep halves with two
// register sets, so the fragments of the next half are read while the MFMAs
// of the current one run, and one barrier per stage publishes the next stage
// and frees a buffer for a later one.  Expert row ranges come from the layout (off_e and cnt_e, or e*C and
// min(cnt_e, C) when padded); each block finds its (expert, row tile) from
// the per-expert tile counts, so the grid is sized without reading anything
// back to the host.
#include "mlp_impl.hpp"
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

template <bool UP, int TM, int NR>
__global__ __launch_bounds__(kThreads) void mlp_kernel(MlpArgs a) {
    mlp_block<UP, TM, NR>(a, blockIdx.x);
}

template <bool UP, int TM, int NR>
hipError_t launch_mlp(const MlpArgs& a, hipStream_t s) {
    const size_t lds = lds_bytes_for<TM>(a.K, a.E, NR);
    MlpArgs g = a;
    const unsigned blocks = mlp_grid<UP, TM>(g);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((mlp_kernel<UP, TM, NR>), dim3(blocks), dim3(kThreads), lds, s, g);
    return hipGetLastError();
}

template <bool UP>
hipError_t launch_pick(const MlpArgs& a, hipStream_t s) {
    const int tm = pick_tm(a.N, a.E), nr = pick_nr(tm, a.K, a.E);
    if (tm == 4) return launch_mlp<UP, 4, 2>(a, s);
    return nr == 3 ? launch_mlp<UP, 2, 3>(a, s) : launch_mlp<UP, 2, 2>(a, s);
}

template <bool UP>
const void* kernel_for(int tm, int nr) {
    if (tm == 4) return (const void*)mlp_kernel<UP, 4, 2>;
    return nr == 3 ? (const void*)mlp_kernel<UP, 2, 3> : (const void*)mlp_kernel<UP, 2, 2>;
}

size_t lds_bytes_tm(int tm, int K, int E, int nr) {
    return tm == 4 ? lds_bytes_for<4>(K, E, nr) : lds_bytes_for<2>(K, E, nr);
}

}  // namespace

size_t expert_mlp_lds_bytes(int N, int K, int E) {
    const int tm = pick_tm(N, E);
    return lds_bytes_tm(tm, K, E, pick_nr(tm, K, E));
}

// Raises the kernels' dynamic-LDS limit above the 64 KiB default (the
// attribute belongs to the function on the current device).
hipError_t prepare_expert_mlp(bool up, int N, int K, int E) {
    const int tm = pick_tm(N, E), nr = pick_nr(tm, K, E);
    const size_t lds = lds_bytes_tm(tm, K, E, nr);
    const void* f = up ? kernel_for<true>(tm, nr) : kernel_for<false>(tm, nr);
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
