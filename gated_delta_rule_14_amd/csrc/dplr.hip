// dplr.hip -- the general diagonal-plus-low-rank (DPLR) recurrence
// ("Diagonal-Plus-Low-Rank Matrices and Kimi Delta Attention", sections 1 and
// 3):
//
//     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,
//
// with two independent low-rank directions a_t, b_t (KDA binds them to the
// key: a_t = beta_t k_t, b_t = k_t * alpha_t) and the decay
// alpha_t = exp(g_min * sigmoid(z_t)) of the "KDA Recurrence" problem.
//
// Per token, with c = S_{t-1}^T b_t (the row the low-rank term erases, read
// from the state before the update):
//     S_t = Diag(alpha) S_{t-1} - a c^T + k v^T
//     o   = S_t^T q = (Diag(alpha) S_{t-1})^T q - (a . q) c + (k . q) v
// so one pass over the old state gives both column sums (b-weighted and
// alpha q-weighted) and the two dot products, and the update follows.
//
//  * dplr_seq_kernel: a whole sequence per (batch, head), the fp32 state in
//    registers (the thread mapping of the decode step: a float4 of value
//    columns over d_k / NRG rows), one workgroup barrier per token (column
//    sums through two alternating LDS buffers), next token's inputs loaded
//    while the current one is processed.
//  * dplr_step_kernel: one token for every (batch, head), the state read from
//    and written back to HBM once (the decode step).
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace dplrk {

template <class E, int DK, int DV, int NTH>
struct Tok {
    static constexpr int NQ = DV / 4, NRG = NTH / NQ, R = DK / NRG;
    static_assert(NQ * NRG == NTH && R * NRG == DK, "bad DPLR tiling");
    E z[R], k[R], q[R], a[R], b[R], v[4];
};

template <class E, int DK, int DV, int NTH>
__device__ __forceinline__ void load_tok(Tok<E, DK, DV, NTH>& t, const E* __restrict__ q, const E* __restrict__ k,
                                         const E* __restrict__ v, const E* __restrict__ z, const E* __restrict__ a,
                                         const E* __restrict__ b, size_t row, int rg, int cq) {
    typedef Tok<E, DK, DV, NTH> T;
#pragma unroll
    for (int i = 0; i < T::R; ++i) {
        const size_t c = row * DK + rg + i * T::NRG;
        t.z[i] = z[c];
        t.k[i] = k[c];
        t.q[i] = q[c];
        t.a[i] = a[c];
        t.b[i] = b[c];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) t.v[j] = v[row * DV + cq * 4 + j];
}

// One token on the register-held rows s: partial column sums into LDS
// buffer `par`, one barrier, then o (returned for row group 0) and the update.
template <class E, int DK, int DV, int NTH, bool RAW_BARRIER>
__device__ __forceinline__ f32x4 token(f32x4 (&s)[DK / (NTH / (DV / 4))], const Tok<E, DK, DV, NTH>& t, float g_min,
                                       float (*red_b)[DV], float (*red_q)[DV], float (*red_s)[2], int rg, int cq) {
    typedef Tok<E, DK, DV, NTH> T;
    float al[T::R], ar[T::R], kr[T::R];
    f32x4 pb = zero4(), pq = zero4();
    float aq = 0.f, kq = 0.f;
#pragma unroll
    for (int i = 0; i < T::R; ++i) {
        al[i] = __expf(g_min * sigmoidf_(to_f32(t.z[i])));
        ar[i] = to_f32(t.a[i]);
        kr[i] = to_f32(t.k[i]);
        const float bi = to_f32(t.b[i]), qi = to_f32(t.q[i]);
        pb += s[i] * bi;
        pq += s[i] * (al[i] * qi);
        aq += ar[i] * qi;
        kq += kr[i] * qi;
    }
    *reinterpret_cast<f32x4*>(&red_b[rg][cq * 4]) = pb;
    *reinterpret_cast<f32x4*>(&red_q[rg][cq * 4]) = pq;
    if (cq == 0) {
        red_s[rg][0] = aq;
        red_s[rg][1] = kq;
    }
    if constexpr (RAW_BARRIER) {
        // a workgroup barrier that leaves the next token's global loads in
        // flight (__syncthreads would wait for them): the wavefront-scope
        // fences only keep the compiler from moving LDS accesses across it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the partials are in LDS
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        __syncthreads();
    }
    f32x4 c = zero4(), d = zero4();
    float aqt = 0.f, kqt = 0.f;
#pragma unroll
    for (int g = 0; g < T::NRG; ++g) {
        c += *reinterpret_cast<const f32x4*>(&red_b[g][cq * 4]);
        d += *reinterpret_cast<const f32x4*>(&red_q[g][cq * 4]);
        aqt += red_s[g][0];
        kqt += red_s[g][1];
    }
    f32x4 vv, ov;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        vv[j] = to_f32(t.v[j]);
        ov[j] = d[j] - aqt * c[j] + kqt * vv[j];
    }
#pragma unroll
    for (int i = 0; i < T::R; ++i) s[i] = s[i] * al[i] - ar[i] * c + kr[i] * vv;
    return ov;
}

template <class E, int DK, int DV, int NTH>
__global__ __launch_bounds__(NTH) void dplr_seq_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                       const E* __restrict__ v, const E* __restrict__ z,
                                                       const E* __restrict__ a, const E* __restrict__ b, float g_min,
                                                       const float* s0, E* __restrict__ o, float* s_final, int T,
                                                       int H) {
    typedef Tok<E, DK, DV, NTH> TK;
    constexpr int NQ = TK::NQ, NRG = TK::NRG, R = TK::R;
    __shared__ float red_b[2][NRG][DV];
    __shared__ float red_q[2][NRG][DV];
    __shared__ float red_s[2][NRG][2];
    const int tid = threadIdx.x, cq = tid % NQ, rg = tid / NQ;
    const size_t bh = blockIdx.x, bb = bh / H, hh = bh % H;
    f32x4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        s[i] = s0 ? *(reinterpret_cast<const f32x4*>(s0 + bh * DK * DV + (size_t)(rg + i * NRG) * DV) + cq) : zero4();
    TK cur, nxt;
    if (T > 0) load_tok<E, DK, DV, NTH>(cur, q, k, v, z, a, b, (bb * T) * H + hh, rg, cq);
    for (int t = 0; t < T; ++t) {
        const int par = t & 1;
        load_tok<E, DK, DV, NTH>(nxt, q, k, v, z, a, b, (bb * T + min(t + 1, T - 1)) * H + hh, rg, cq);
        const f32x4 ov = token<E, DK, DV, NTH, true>(s, cur, g_min, red_b[par], red_q[par], red_s[par], rg, cq);
        if (rg == 0) {
            E* oh = o + ((bb * T + t) * H + hh) * DV + cq * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) oh[j] = from_f32<E>(ov[j]);
        }
        cur = nxt;
    }
    if (s_final) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            *(reinterpret_cast<f32x4*>(s_final + bh * DK * DV + (size_t)(rg + i * NRG) * DV) + cq) = s[i];
    }
}

template <class E, int DK, int DV, int NTH>
__global__ __launch_bounds__(NTH) void dplr_step_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                        const E* __restrict__ v, const E* __restrict__ z,
                                                        const E* __restrict__ a, const E* __restrict__ b,
                                                        float g_min, float* __restrict__ state, E* __restrict__ o) {
    typedef Tok<E, DK, DV, NTH> TK;
    constexpr int NQ = TK::NQ, NRG = TK::NRG, R = TK::R;
    __shared__ float red_b[NRG][DV];
    __shared__ float red_q[NRG][DV];
    __shared__ float red_s[NRG][2];
    const int tid = threadIdx.x, cq = tid % NQ, rg = tid / NQ;
    const size_t bh = blockIdx.x;
    float* S = state + bh * DK * DV;
    f32x4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg + i * NRG) * DV) + cq);
    TK tok;
    load_tok<E, DK, DV, NTH>(tok, q, k, v, z, a, b, bh, rg, cq);
    const f32x4 ov = token<E, DK, DV, NTH, false>(s, tok, g_min, red_b, red_q, red_s, rg, cq);
    if (rg == 0) {
        E* oh = o + bh * DV + cq * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) oh[j] = from_f32<E>(ov[j]);
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
        __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (size_t)(rg + i * NRG) * DV) + cq);
}

template <class E, int DK, int DV>
hipError_t launch_t(const DplrArgs& x) {
    constexpr int NTH = (DK == 128 && DV == 128) ? 512 : 256;
    hipStream_t st = (hipStream_t)x.stream;
    if (x.step)
        hipLaunchKernelGGL((dplr_step_kernel<E, DK, DV, NTH>), dim3(x.B * x.H), dim3(NTH), 0, st, (const E*)x.q,
                           (const E*)x.k, (const E*)x.v, (const E*)x.z, (const E*)x.a, (const E*)x.b, x.g_min,
                           x.s_final, (E*)x.o);
    else
        hipLaunchKernelGGL((dplr_seq_kernel<E, DK, DV, NTH>), dim3(x.B * x.H), dim3(NTH), 0, st, (const E*)x.q,
                           (const E*)x.k, (const E*)x.v, (const E*)x.z, (const E*)x.a, (const E*)x.b, x.g_min, x.s0,
                           (E*)x.o, x.s_final, x.T, x.H);
    return hipGetLastError();
}

template <class E>
hipError_t launch_e(const DplrArgs& x) {
    if (x.dk == 128 && x.dv == 128) return launch_t<E, 128, 128>(x);
    if (x.dk == 128 && x.dv == 64) return launch_t<E, 128, 64>(x);
    if (x.dk == 64 && x.dv == 128) return launch_t<E, 64, 128>(x);
    return launch_t<E, 64, 64>(x);
}

}  // namespace dplrk

hipError_t launch_dplr(const DplrArgs& x) { return x.bf16 ? dplrk::launch_e<bf16>(x) : dplrk::launch_e<float>(x); }

}  // namespace kda
