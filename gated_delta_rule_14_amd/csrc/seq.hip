// seq.hip -- token-sequential prefill: the recurrence of Eq. 1 (Kimi Linear
// tech report, section 3) taken one token at a time over a whole sequence,
// with the decay and readout of the "KDA Recurrence" problem statement.
//
// The chunkwise kernels factor each decay product e^{G_r - G_i} inside a
// 64-token chunk into per-row and per-column factors around 16-row block
// references.  A factor spans up to eight tokens of decay, so it can reach
// 2^{8 |g_min| log2 e}; for g_min >= -8 that is at most 2^93, finite, and the
// parts lost where a partner factor underflows stay below 2^-40.  For
// stronger decay bounds the prefill calls run this kernel instead: every
// step uses alpha_t itself, which is exact for any g_min < 0.
//
// One workgroup per (b, h) keeps the fp32 d_k x d_v state in registers for
// the whole sequence, with the thread mapping of the decode step (decode.hip):
// thread t owns a float4 of value columns over d_k / NRG rows, NRG apart.
// Per token, the step order of the agentlenshq blog's fused recurrent kernel:
//   S' = Diag(alpha) S,  p = S'^T k,  r = beta (v - p),  S = S' + k r^T,
//   o = S^T q = S'^T q + (k . q) r.
// The column sums go through LDS in two alternating buffers, so a token
// costs one workgroup barrier; the next token's inputs are loaded while the
// current one is processed.  GATED also applies the layer's output epilogue
// (RMS normalisation over d_v with eps inside the root, times sigmoid(gate))
// to each token's fp32 read-out.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

template <class E, int DK, int DV, int NTH, bool GATED, class Y>
__global__ __launch_bounds__(NTH) void seq_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ z,
    const E* __restrict__ beta, float g_min, const float* s0, E* __restrict__ o,
    float* s_final, const E* __restrict__ gate, float eps, Y* __restrict__ y, int T, int H) {
    constexpr int NQ = DV / 4;       // column quads
    constexpr int NRG = NTH / NQ;    // row groups
    constexpr int R = DK / NRG;      // rows per thread
    static_assert(NQ * NRG == NTH && R * NRG == DK, "bad tiling");

    __shared__ float red_p[2][NRG][DV];
    __shared__ float red_q[2][NRG][DV];
    __shared__ float red_kq[2][NRG];

    const int tid = threadIdx.x;
    const int cq = tid % NQ;
    const int rg = tid / NQ;
    const size_t bh = blockIdx.x;
    const size_t b = bh / H, h = bh % H;

    f32x4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        s[i] = s0 ? *(reinterpret_cast<const f32x4*>(s0 + bh * DK * DV + (size_t)(rg + i * NRG) * DV) + cq) : zero4();

    // raw inputs of one token, as this thread needs them
    E zc[R], kc[R], qc[R], vc[4], gc[4], bc;
    auto fetch = [&](int t) {
        const size_t rt = ((size_t)b * T + t) * H + h;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int c = rg + i * NRG;
            zc[i] = z[rt * DK + c];
            kc[i] = k[rt * DK + c];
            qc[i] = q[rt * DK + c];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) vc[j] = v[rt * DV + cq * 4 + j];
        if constexpr (GATED) {
#pragma unroll
            for (int j = 0; j < 4; ++j) gc[j] = gate[rt * DV + cq * 4 + j];
        }
        bc = beta[rt];
    };
    if (T > 0) fetch(0);

    for (int t = 0; t < T; ++t) {
        const int par = t & 1;
        float a[R], kr[R], qr[R], vr[4], gr[4];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            a[i] = __expf(g_min * sigmoidf_(to_f32(zc[i])));
            kr[i] = to_f32(kc[i]);
            qr[i] = to_f32(qc[i]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vr[j] = to_f32(vc[j]);
            gr[j] = GATED ? to_f32(gc[j]) : 0.f;
        }
        const float bt = to_f32(bc);
        fetch(min(t + 1, T - 1));   // the next token (unconditional, in bounds)

        f32x4 pk = zero4(), pq = zero4();
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            s[i] *= a[i];
            pk += s[i] * kr[i];
            pq += s[i] * qr[i];
            kq += kr[i] * qr[i];
        }
        *reinterpret_cast<f32x4*>(&red_p[par][rg][cq * 4]) = pk;
        *reinterpret_cast<f32x4*>(&red_q[par][rg][cq * 4]) = pq;
        if (cq == 0) red_kq[par][rg] = kq;
        __syncthreads();

        f32x4 p = zero4(), sq = zero4();
        float kqt = 0.f;
#pragma unroll
        for (int g = 0; g < NRG; ++g) {
            p += *reinterpret_cast<const f32x4*>(&red_p[par][g][cq * 4]);
            sq += *reinterpret_cast<const f32x4*>(&red_q[par][g][cq * 4]);
            kqt += red_kq[par][g];
        }
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = bt * (vr[j] - p[j]);

        if (rg == 0) {
            const size_t rt = ((size_t)b * T + t) * H + h;
            f32x4 ov;
#pragma unroll
            for (int j = 0; j < 4; ++j) ov[j] = sq[j] + kqt * r[j];
            if (o) {
#pragma unroll
                for (int j = 0; j < 4; ++j) o[rt * DV + cq * 4 + j] = from_f32<E>(ov[j]);
            }
            if constexpr (GATED) {
                // row group 0 is lanes 0 .. NQ-1 of wave 0
                float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
                for (int off = NQ / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, NQ);
                const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float sg = sizeof(E) == 4 ? 1.0f / (1.0f + expf(-gr[j])) : sigmoidf_(gr[j]);
                    y[rt * DV + cq * 4 + j] = from_f32<Y>(ov[j] * inv * sg);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) s[i] += kr[i] * r;
    }
    if (s_final) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            *(reinterpret_cast<f32x4*>(s_final + bh * DK * DV + (size_t)(rg + i * NRG) * DV) + cq) = s[i];
    }
}

template <class E, int DK, int DV>
static hipError_t launch_seq_t(const ChunkArgs& a) {
    constexpr int NTH = (DK == 128 && DV == 128) ? 512 : 256;
    const dim3 grid(a.B * a.H), block(NTH);
    hipStream_t st = (hipStream_t)a.stream;
    if (!a.gate)
        hipLaunchKernelGGL((seq_fwd_kernel<E, DK, DV, NTH, false, E>), grid, block, 0, st, (const E*)a.q,
                           (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.s0, (E*)a.o,
                           a.s_final, (const E*)nullptr, 0.f, (E*)nullptr, a.T, a.H);
    else
        hipLaunchKernelGGL((seq_fwd_kernel<E, DK, DV, NTH, true, E>), grid, block, 0, st, (const E*)a.q,
                           (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.s0, (E*)a.o,
                           a.s_final, (const E*)a.gate, a.eps, (E*)a.y, a.T, a.H);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_seq_e(const ChunkArgs& a) {
    if (a.dk == 128 && a.dv == 128) return launch_seq_t<E, 128, 128>(a);
    if (a.dk == 128 && a.dv == 64) return launch_seq_t<E, 128, 64>(a);
    if (a.dk == 64 && a.dv == 128) return launch_seq_t<E, 64, 128>(a);
    return launch_seq_t<E, 64, 64>(a);
}

hipError_t launch_seq(const ChunkArgs& a) { return a.bf16 ? launch_seq_e<bf16>(a) : launch_seq_e<float>(a); }

}  // namespace kda
