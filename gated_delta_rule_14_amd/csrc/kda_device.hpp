// kda_device.hpp -- device-side building blocks shared by the libkda kernels
// (gfx950 / CDNA4, wave64).
//
//  * element types: fp32 and bf16 (__bf16, converted round-to-nearest-even);
//  * 16x16 MFMA tiles with fp32 accumulation: v_mfma_f32_16x16x32_bf16 for
//    bf16 operands and v_mfma_f32_16x16x4_f32 for fp32 operands;
//  * fragment loaders for operands stored "K-contiguous" (each row of the
//    A operand and each column of the B operand is contiguous along the
//    contraction index), which is how every LDS tile in libkda is laid out.
//
// Lane layout of a 16x16 tile on a 64-wide wavefront (lane l):
//   A operand (16 x K):  row l%16, contraction indices [(l/16)*KPL, +KPL)
//   B operand (K x 16):  col l%16, contraction indices [(l/16)*KPL, +KPL)
//   C / D (16 x 16):     col l%16, rows 4*(l/16) + e, e = 0..3
// where KPL is 8 for bf16 (K = 32 per instruction) and 1 for fp32 (K = 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;   // 16-byte raw vector

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// Wave index, made provably wave-uniform so that it lives in an SGPR: table
// lookups become scalar loads and branches on it become scalar branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------- MFMA
template <class CT> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int KSTEP = 32;   // contraction length per instruction
    static constexpr int KPL = 8;      // contraction elements per lane
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag from_floats(const float* v) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
        return f;
    }
    static __device__ __forceinline__ void to_floats(frag f, float* v) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)f[i];
    }
};

template <> struct Mfma<float> {
    static constexpr int KSTEP = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag from_floats(const float* v) { return v[0]; }
    static __device__ __forceinline__ void to_floats(frag f, float* v) { v[0] = f; }
};

// Fragment of a K-contiguous tile: element (row0 + l%16, k0 + (l/16)*KPL + j).
// `ld` is the row stride in elements; for bf16 the address must be 16-byte
// aligned (ld and k0 multiples of 8).
template <class CT>
__device__ __forceinline__ typename Mfma<CT>::frag load_frag(const CT* base, int ld, int row0, int k0, int l) {
    const CT* p = base + (size_t)(row0 + (l & 15)) * ld + k0 + (l >> 4) * Mfma<CT>::KPL;
    return *reinterpret_cast<const typename Mfma<CT>::frag*>(p);
}
template <class CT>
__device__ __forceinline__ typename Mfma<CT>::frag load_frag(const CT* base, int ld, int row0, int k0) {
    return load_frag<CT>(base, ld, row0, k0, lane_id());
}

// An opaque copy of x: values computed from it inside a loop are not hoisted
// into the preheader, where they would hold registers across the whole loop.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Same addressing, from an fp32 tile, converted to the operand type.
template <class CT>
__device__ __forceinline__ typename Mfma<CT>::frag load_frag_f32(const float* base, int ld, int row0, int k0) {
    const int l = lane_id();
    const float* p = base + (size_t)(row0 + (l & 15)) * ld + k0 + (l >> 4) * Mfma<CT>::KPL;
    float v[Mfma<CT>::KPL];
#pragma unroll
    for (int j = 0; j < Mfma<CT>::KPL; ++j) v[j] = p[j];
    return Mfma<CT>::from_floats(v);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row / column of accumulator element e held by this lane.
__device__ __forceinline__ int acc_row(int e) { return 4 * (lane_id() >> 4) + e; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

// v_rcp_f32 (1 ulp) instead of a correctly rounded IEEE division
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Four / eight consecutive elements, converted from / to fp32.  p must be
// aligned to the access size (8 or 16 bytes for bf16, 16 or 32 for fp32).
template <class CT> __device__ __forceinline__ void store4(CT* p, f32x4 v);
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
    *reinterpret_cast<f32x4*>(p) = v;
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, f32x4 v) {
    bf16x4 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (bf16)v[i];
    *reinterpret_cast<bf16x4*>(p) = b;
}
template <class CT> __device__ __forceinline__ f32x4 load4(const CT* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
// Two consecutive elements of type E, loaded / stored as one access.
template <class E> struct Pair;
template <> struct Pair<float> { typedef f32x2 type; };
template <> struct Pair<bf16> { typedef bf16x2 type; };
template <class E> __device__ __forceinline__ typename Pair<E>::type load2(const E* p) {
    return *reinterpret_cast<const typename Pair<E>::type*>(p);
}
template <class E> __device__ __forceinline__ void store2(E* p, float a, float b) {
    typename Pair<E>::type v;
    v[0] = from_f32<E>(a);
    v[1] = from_f32<E>(b);
    *reinterpret_cast<typename Pair<E>::type*>(p) = v;
}

// Raw (unconverted) four-element vectors, for register prefetch: converting
// at load time would make the load's consumer wait for it.
template <class CT> struct Raw4;
template <> struct Raw4<float> { typedef f32x4 type; };
template <> struct Raw4<bf16> { typedef bf16x4 type; };
template <class CT> __device__ __forceinline__ typename Raw4<CT>::type load_raw4(const CT* p) {
    return *reinterpret_cast<const typename Raw4<CT>::type*>(p);
}
__device__ __forceinline__ f32x4 widen4(f32x4 v) { return v; }
__device__ __forceinline__ f32x4 widen4(bf16x4 b) { return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]}; }

template <class CT> __device__ __forceinline__ void store8(CT* p, const float* v) {
    store4<CT>(p, f32x4{v[0], v[1], v[2], v[3]});
    store4<CT>(p + 4, f32x4{v[4], v[5], v[6], v[7]});
}
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, const float* v) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = b;
}

}  // namespace kda
