// scalar_gate.hip -- the Gated DeltaNet special case of the operator: one
// decay logit per (token, head) instead of one per key channel, so that
// alpha_t is a scalar and Diag(alpha_t) = alpha_t I ("Kimi Linear" tech
// report, section 3: KDA refines the scalar gate of Gated DeltaNet into a
// channel-wise one; "Diagonal-Plus-Low-Rank Matrices and Kimi Delta
// Attention": a uniform alpha is the scalar-decay case).
//
// The prefill runs through the same kernels as the channel-wise operator.
// The pipelined bf16 kernels (d_k = d_v = 128) read the scalar logit directly
// and form each row's decay factors once (seg.hip, SG); elsewhere
// broadcast_gate_kernel writes each scalar logit across the d_k channels of
// a workspace buffer, which then serves as z.  Decode reads the scalar
// directly (decode.hip).
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

// zfull[r * dk + c] = zs[r] for r < rows, c < dk; 16 bytes per store.
template <class E>
__global__ __launch_bounds__(256) void broadcast_gate_kernel(const E* __restrict__ zs, E* __restrict__ zfull,
                                                             size_t rows, int dk) {
    constexpr int PER = 16 / sizeof(E);                  // elements per 16-byte store
    const size_t vecs_per_row = (size_t)dk / PER;
    const size_t n = rows * vecs_per_row;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const E x = zs[i / vecs_per_row];
        if constexpr (sizeof(E) == 2) {
            bf16x8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = x;
            reinterpret_cast<bf16x8*>(zfull)[i] = v;
        } else {
            reinterpret_cast<f32x4*>(zfull)[i] = f32x4{x, x, x, x};
        }
    }
}

hipError_t launch_broadcast_gate(const void* zs, void* zfull, size_t rows, int dk, bool is_bf16, void* stream) {
    if (rows == 0) return hipSuccess;
    const size_t vecs = rows * (size_t)dk / (is_bf16 ? 8 : 4);
    size_t blocks = (vecs + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipStream_t st = (hipStream_t)stream;
    if (is_bf16)
        hipLaunchKernelGGL((broadcast_gate_kernel<bf16>), dim3((unsigned)blocks), dim3(256), 0, st, (const bf16*)zs,
                           (bf16*)zfull, rows, dk);
    else
        hipLaunchKernelGGL((broadcast_gate_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, st, (const float*)zs,
                           (float*)zfull, rows, dk);
    return hipGetLastError();
}

}  // namespace kda
