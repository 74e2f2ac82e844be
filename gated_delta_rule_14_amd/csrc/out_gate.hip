// out_gate.hip -- kda_out_gate: the KDA output epilogue.
//
// "KDA Recurrence" problem statement (and its first worked example): for
// every (batch, token, head), normalise the head's d_v outputs by their RMS
// (eps inside the square root, no learnable weight), multiply by the sigmoid
// of the output-gate logits, concatenate the heads to width H*d_v, then
// optionally project: out = y W^T with W of shape (d_model, H*d_v), no bias.
//
//  * gate_kernel: one row of d_v values per 1..2 dozen lanes, 16-byte loads,
//    shuffle reduction of the sum of squares; HBM-bound elementwise work.
//  * the projection is libkda's own GEMM (gemm.hip) on the gated rows, which
//    the gate kernel writes in bf16 to the workspace.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

// Row `row` (d_v values of one token and head), lane `sub` of its LPR lanes:
// each lane reads its 8 values of o and of the gate, then writes its 8 values
// of y at the same offset, so o and y may be the same memory.
template <class E, int DV>
__device__ __forceinline__ void gate_row(const E* o, const E* gate, float eps, E* y, size_t row, int sub) {
    constexpr int LPR = DV / 8;              // lanes per row, 8 values per lane
    const size_t base = row * DV + sub * 8;
    float x[8], g[8];
    if constexpr (sizeof(E) == 2) {
        // non-temporal: every byte is touched once (279 -> 256 us on the
        // 8 x 8192 x 32-head rows, one box)
        const bf16x8 xv = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(o + base));
        const bf16x8 gv = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(gate + base));
#pragma unroll
        for (int j = 0; j < 8; ++j) { x[j] = (float)xv[j]; g[j] = (float)gv[j]; }
    } else {
        const f32x4* xp = reinterpret_cast<const f32x4*>(o + base);
        const f32x4* gp = reinterpret_cast<const f32x4*>(gate + base);
        const f32x4 x0 = xp[0], x1 = xp[1], g0 = gp[0], g1 = gp[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) { x[j] = x0[j]; x[4 + j] = x1[j]; g[j] = g0[j]; g[4 + j] = g1[j]; }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, LPR);
    const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
    if constexpr (sizeof(E) == 2) {
        bf16x8 out;
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = (bf16)(x[j] * inv * sigmoidf_(g[j]));
        __builtin_nontemporal_store(out, reinterpret_cast<bf16x8*>(y + base));
    } else {
        f32x4 y0, y1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            y0[j] = x[j] * inv * (1.0f / (1.0f + expf(-g[j])));
            y1[j] = x[4 + j] * inv * (1.0f / (1.0f + expf(-g[4 + j])));
        }
        reinterpret_cast<f32x4*>(y + base)[0] = y0;
        reinterpret_cast<f32x4*>(y + base)[1] = y1;
    }
}

template <class E, int DV>
__global__ __launch_bounds__(256) void gate_kernel(const E* __restrict__ o, const E* __restrict__ gate,
                                                   float eps, E* __restrict__ y, size_t rows) {
    constexpr int LPR = DV / 8;              // lanes per row, 8 values per lane
    constexpr int RPB = 256 / LPR;           // rows per block per iteration
    const int tid = threadIdx.x;
    for (size_t row = (size_t)blockIdx.x * RPB + tid / LPR; row < rows; row += (size_t)gridDim.x * RPB)
        gate_row<E, DV>(o, gate, eps, y, row, tid % LPR);
}

// The epilogue on the rows of tokens [0, t_a) and [t_b, T) of each of the
// sequences (bf16, d_v = 128): the rows that the split prefill plan's full
// expands leave to it.  o may be y.
__global__ __launch_bounds__(256) void gate_ends_kernel(const bf16* o, const bf16* __restrict__ gate, float eps,
                                                        bf16* y, int T, int H, int t_a, int t_b, size_t rows) {
    constexpr int LPR = 16, RPB = 256 / LPR;
    const int tid = threadIdx.x;
    const size_t ra = (size_t)t_a * H, per_b = ra + (size_t)(T - t_b) * H;
    for (size_t r = (size_t)blockIdx.x * RPB + tid / LPR; r < rows; r += (size_t)gridDim.x * RPB) {
        const size_t b = r / per_b, loc = r % per_b;
        const size_t row = b * T * H + (loc < ra ? loc : (size_t)t_b * H + (loc - ra));
        gate_row<bf16, 128>(o, gate, eps, y, row, tid % LPR);
    }
}

hipError_t launch_gate_ends(const void* o, const void* gate, float eps, void* y, int B, int T, int H, int t_a, int t_b,
                            void* stream) {
    const size_t rows = (size_t)B * ((size_t)t_a + (size_t)(T - t_b)) * H;
    size_t blocks = (rows + 15) / 16;
    if (blocks > (size_t(1) << 22)) blocks = size_t(1) << 22;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(gate_ends_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const bf16*)o,
                       (const bf16*)gate, eps, (bf16*)y, T, H, t_a, t_b, rows);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_gate(const void* o, const void* gate, float eps, void* y, size_t rows, int dv,
                              hipStream_t st) {
    const int lpr = dv / 8, rpb = 256 / lpr;
    size_t blocks = (rows + rpb - 1) / rpb;
    // One pass over the rows when it fits: a grid-stride second pass measured
    // about 12% slower on 2M rows of 128 values than one block per 16 rows.
    if (blocks > (size_t(1) << 22)) blocks = size_t(1) << 22;
    if (blocks == 0) return hipSuccess;
    if (dv == 128)
        hipLaunchKernelGGL((gate_kernel<E, 128>), dim3((unsigned)blocks), dim3(256), 0, st, (const E*)o,
                           (const E*)gate, eps, (E*)y, rows);
    else
        hipLaunchKernelGGL((gate_kernel<E, 64>), dim3((unsigned)blocks), dim3(256), 0, st, (const E*)o,
                           (const E*)gate, eps, (E*)y, rows);
    return hipGetLastError();
}

static size_t y_bytes(int B, int T, int H, int dv) { return ((size_t)B * T * H * dv * 2 + 255) / 256 * 256; }

size_t gate_workspace_bytes(int B, int T, int H, int dv, int d_model, bool bf16, bool proj) {
    (void)bf16;
    if (!proj) return 0;
    // gated activations y (bf16), then the GEMM's scratch
    return y_bytes(B, T, H, dv) + projection_scratch_bytes(B * T, d_model, H * dv);
}

hipError_t launch_out_gate(const GateArgs& a) {
    hipStream_t st = (hipStream_t)a.stream;
    const size_t rows = (size_t)a.B * a.T * a.H;
    if (!a.w) {
        return a.bf16 ? launch_gate<bf16>(a.o, a.gate, a.eps, a.y, rows, a.dv, st)
                      : launch_gate<float>(a.o, a.gate, a.eps, a.y, rows, a.dv, st);
    }
    hipError_t err = launch_gate<bf16>(a.o, a.gate, a.eps, a.workspace, rows, a.dv, st);
    if (err != hipSuccess) return err;
    void* lws = (unsigned char*)a.workspace + y_bytes(a.B, a.T, a.H, a.dv);
    return launch_projection(a.workspace, a.w, a.y, a.B * a.T, a.d_model, a.H * a.dv, lws, a.stream);
}

}  // namespace kda
