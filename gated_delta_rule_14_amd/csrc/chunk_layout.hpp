// chunk_layout.hpp -- the per-chunk workspace layouts shared by the
// workspace-based chunk kernels (chunk.hip: the fp32 prefill and the forward
// half of kda_chunk_bwd; bwd_chunk.hip: the backward's own kernels).
#pragma once

#include "kda_device.hpp"

namespace kda {

constexpr int C = 64;     // chunk length
constexpr int SUB = 16;   // block size of the triangular solve and of A / M

template <class E> struct Compute { typedef bf16 type; };
template <> struct Compute<float> { typedef float type; };

// exp for decay factors: libm-accurate on the fp32 path, the hardware
// exp2-based one on the bf16 path.
template <class E> __device__ __forceinline__ float dexp(float x) { return __expf(x); }
template <> __device__ __forceinline__ float dexp<float>(float x) { return expf(x); }
template <class E> __device__ __forceinline__ float dsigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + dexp<E>(-x)); }

constexpr size_t align16(size_t x) { return (x + 15) / 16 * 16; }
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// Workspace block of one (b, h, chunk), offsets in elements of the compute
// type CT; every part starts on a 16-byte boundary.
template <class CT, int DK, int DV>
struct Ws {
    static constexpr size_t W = 0;                     // (C, DK)  row-major
    static constexpr size_t UT = W + (size_t)C * DK;   // (DV, C)  U transposed
    static constexpr size_t M = UT + (size_t)DV * C;   // (C, C)
    static constexpr size_t QG = M + (size_t)C * C;    // (C, DK)  q * e^{G}
    static constexpr size_t KGT = QG + (size_t)C * DK; // (DK, C)  (k * e^{G_C - G})^T
    static constexpr size_t END = KGT + (size_t)DK * C;
    static constexpr size_t BYTES = END * sizeof(CT) + DK * sizeof(float);  // + e^{G_C} fp32
};

// The same chunk's operands as the backward's reverse chunk recurrence
// contracts them (kda_chunk_bwd): M^T, K e^{G_C - G} row-major, (Q e^G)^T and
// W^T; with bf16 tokens also T^T (T = (I + diag(beta) Ab)^{-1}) and Ab =
// tril_-1(Kg Kt^T) for the per-chunk gradients.  Written by the intra-chunk
// kernel only when it runs for the backward.
template <class CT, int DK, int DV>
struct WsB {
    static constexpr size_t MT = 0;                     // (C, C)   M^T
    static constexpr size_t KC = MT + (size_t)C * C;    // (C, DK)  k * e^{G_C - G}
    static constexpr size_t QGT = KC + (size_t)C * DK;  // (DK, C)  (q * e^G)^T
    static constexpr size_t WT = QGT + (size_t)DK * C;  // (DK, C)  W^T
    static constexpr size_t TT = WT + (size_t)DK * C;   // (C, C)   T^T      (bf16 tokens)
    static constexpr size_t AB = TT + (size_t)C * C;    // (C, C)   Ab       (bf16 tokens)
    static constexpr size_t END = AB + (size_t)C * C;
    static constexpr size_t BYTES = END * sizeof(CT);
};

}  // namespace kda
