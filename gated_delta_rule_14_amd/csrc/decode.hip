// decode.hip -- kda_recurrent_step: one token of the KDA recurrence for every
// (batch, head), with the fp32 state streamed through registers.
//
// Per (b, h), following the token step of the fused recurrent decode kernel
// described in the agentlenshq KDA blog (efficient-execution section) and the
// readout rule of the "KDA Recurrence" problem (read the updated state):
//   alpha = exp(g_min * sigmoid(z))          per key channel
//   S'    = Diag(alpha) S
//   p     = S'^T k,   r = beta (v - p)
//   S     = S' + k r^T                        (written back in place)
//   o     = S^T q = S'^T q + (k . q) r
// which is Eq. 1 of the tech report rearranged exactly.
//
// Work mapping: one workgroup per (b, h) (512 threads for d_k = d_v = 128,
// 256 otherwise).  Thread t owns four
// consecutive value columns (a float4) of DK / NRG rows, the rows of one
// thread being NRG apart so that a wavefront's loads cover whole adjacent
// rows (fully coalesced 16-byte accesses).  The state is read once into
// VGPRs, the two column reductions (p and S'^T q) go through LDS, and the
// updated state is written once.  The kernel is purely HBM-bound: 2 * 4 *
// DK * DV bytes of state traffic against ~7 * DK * DV flops.
//
// kda_recurrent_layer_step runs the same kernel with the output epilogue
// fused (RMS normalisation over d_v times sigmoid(gate)), so that one
// decode token of the whole layer is one launch, plus the projection GEMM
// when one is asked for.
#include "kda_device.hpp"
#include "kda_internal.hpp"

// Threads per (b, h) for d_k = d_v = 128: 512 keeps 32 state values per
// thread, which leaves room for more resident waves than 256 threads do.
#ifndef KDA_DECODE_THREADS
#define KDA_DECODE_THREADS 512
#endif

namespace kda {

// GATED: also the layer's output epilogue on the fp32 read-out o of each
// (b, h): y = o / sqrt(mean(o^2) + eps) * sigmoid(gate), in dtype Y ("KDA
// Recurrence" problem statement); the threads of row group 0, which hold
// the d_v outputs four apiece, reduce the sum of squares by lane shuffles.
// o is written only when it is not NULL.
// ZS: z holds one logit per (b, h), the same for every key channel (the
// scalar-decay case).
template <class E, int DK, int DV, int NTH, bool GATED, class Y, bool ZS = false>
__global__ __launch_bounds__(NTH) void decode_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const E* __restrict__ beta, float g_min,
    float* __restrict__ state, E* __restrict__ o, const E* __restrict__ gate, float eps,
    Y* __restrict__ y) {
    constexpr int NQ = DV / 4;       // column quads
    constexpr int NRG = NTH / NQ;    // row groups
    constexpr int R = DK / NRG;      // rows per thread
    static_assert(NQ * NRG == NTH && R * NRG == DK, "bad decode tiling");

    __shared__ float red_p[NRG][DV];
    __shared__ float red_q[NRG][DV];
    __shared__ float red_kq[NRG];

    const int tid = threadIdx.x;
    const int cq = tid % NQ;
    const int rg = tid / NQ;
    const size_t bh = blockIdx.x;

    float* S = state + bh * DK * DV;
    const E* qh = q + bh * DK;
    const E* kh = k + bh * DK;
    const E* zh = ZS ? z + bh : z + bh * DK;

    f32x4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg + i * NRG) * DV) + cq);

    float kr[R];
    f32x4 pk = zero4(), pq = zero4();
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int c = rg + i * NRG;
        const float zc = to_f32(zh[ZS ? 0 : c]);
        const float a = __expf(g_min * sigmoidf_(zc));
        const float kc = to_f32(kh[c]);
        const float qc = to_f32(qh[c]);
        s[i] *= a;
        pk += s[i] * kc;
        pq += s[i] * qc;
        kq += kc * qc;
        kr[i] = kc;
    }
    *reinterpret_cast<f32x4*>(&red_p[rg][cq * 4]) = pk;
    *reinterpret_cast<f32x4*>(&red_q[rg][cq * 4]) = pq;
    if (cq == 0) red_kq[rg] = kq;
    __syncthreads();

    f32x4 p = zero4(), sq = zero4();
    float kqt = 0.f;
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
        p += *reinterpret_cast<const f32x4*>(&red_p[g][cq * 4]);
        sq += *reinterpret_cast<const f32x4*>(&red_q[g][cq * 4]);
        kqt += red_kq[g];
    }
    const float b = to_f32(beta[bh]);
    const E* vh = v + bh * DV + cq * 4;
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = b * (to_f32(vh[j]) - p[j]);

    if (rg == 0) {
        f32x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = sq[j] + kqt * r[j];
        if (o) {
            E* oh = o + bh * DV + cq * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) oh[j] = from_f32<E>(ov[j]);
        }
        if constexpr (GATED) {
            // row group 0 is lanes 0 .. NQ-1 of wave 0
            float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
            for (int off = NQ / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, NQ);
            const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
            const E* gh = gate + bh * DV + cq * 4;
            Y* yh = y + bh * DV + cq * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float gj = to_f32(gh[j]);
                const float sg = sizeof(E) == 4 ? 1.0f / (1.0f + expf(-gj)) : sigmoidf_(gj);
                yh[j] = from_f32<Y>(ov[j] * inv * sg);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        f32x4 sn = s[i] + kr[i] * r;
        __builtin_nontemporal_store(sn, reinterpret_cast<f32x4*>(S + (size_t)(rg + i * NRG) * DV) + cq);
    }
}

template <class E, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    constexpr int NTH = (DK == 128 && DV == 128) ? KDA_DECODE_THREADS : 256;
    const dim3 grid(a.B * a.H), block(NTH);
    hipStream_t st = (hipStream_t)a.stream;
    if (a.z_scalar)
        hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, NTH, false, E, true>), grid, block, 0, st, (const E*)a.q,
                           (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.state,
                           (E*)a.o, nullptr, 0.f, nullptr);
    else if (!a.gate)
        hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, NTH, false, E>), grid, block, 0, st, (const E*)a.q,
                           (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.state,
                           (E*)a.o, nullptr, 0.f, nullptr);
    else if (a.y_bf16)
        hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, NTH, true, bf16>), grid, block, 0, st, (const E*)a.q,
                           (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.state,
                           (E*)a.o, (const E*)a.gate, a.eps, (bf16*)a.y);
    else
        hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, NTH, true, E>), grid, block, 0, st, (const E*)a.q,
                           (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.state,
                           (E*)a.o, (const E*)a.gate, a.eps, (E*)a.y);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_decode_e(const DecodeArgs& a) {
    if (a.dk == 128 && a.dv == 128) return launch_decode_t<E, 128, 128>(a);
    if (a.dk == 128 && a.dv == 64) return launch_decode_t<E, 128, 64>(a);
    if (a.dk == 64 && a.dv == 128) return launch_decode_t<E, 64, 128>(a);
    return launch_decode_t<E, 64, 64>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
    return a.bf16 ? launch_decode_e<bf16>(a) : launch_decode_e<float>(a);
}

}  // namespace kda
