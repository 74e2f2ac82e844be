// bwd.hip -- gradients of the KDA recurrence (Kimi Linear tech report,
// section 3, Eq. 1, with the decay and readout of the "KDA Recurrence"
// problem statement) with respect to q, k, v, the decay logits z, beta and
// the initial state, for given gradients of the outputs and of the final
// state.  The pages give no gradient formulas; the chain rule through one
// token (S' = Diag(alpha) S, w = v - S'^T k, S_t = S' + beta k w^T,
// o = S_t^T q) gives, with dS the gradient with respect to S_t:
//
//   dq = S_t do,  dS += q do^T,  u = dS^T k,  dbeta = u . w,  dw = beta u,
//   dv = dw,  dk = beta dS w - S' dw,  dS' = dS - k dw^T,
//   dalpha = rowsum(S_{t-1} * dS'),  dz = dalpha alpha g_min sigmoid(z)(1 - sigmoid(z)),
//   dS <- Diag(alpha) dS'   (the gradient with respect to S_{t-1}).
//
// recurrent_bwd_kernel: one workgroup of 4 d_k threads per (batch, head);
// thread (row r, quarter g) holds state row r, columns [g d_v/4, (g+1) d_v/4),
// so that the row sums (dq, dk, dalpha) are two lane exchanges and the
// column sums (S'^T k forward, dS^T k backward) go through LDS.  A forward
// sweep stores the state at the start of every 64-token interval in the
// workspace; the backward sweep then takes the intervals in reverse: it
// recomputes the interval's states forward (storing each token's incoming
// state in the workspace and w in LDS) and steps back through its tokens
// with dS in registers.  Token-sequential: every token costs two workgroup
// barriers in each direction.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwdk {

constexpr int C = 64;   // tokens per stored state

template <int DK, int DV>
struct BLay {
    static constexpr int NTH = 4 * DK;
    static constexpr int SW = DV / 4;           // columns per thread
    static constexpr int RP = DV + 4;           // row pitch of the column-sum partials (floats)
    static constexpr int NPR = NTH / 16;        // partial rows: one per 16-lane group (4 state rows)
    static constexpr int TPC = NTH / DV;        // threads per column in the column sums
    static constexpr int RPT = NPR / TPC;       // partial rows per thread in the column sums
    // one staged token: q, k, alpha, the dz factor (DK each), v or do (DV), beta
    static constexpr int TOK = 4 * DK + DV + 4;
    static constexpr int OFF_RED = 0;                     // [NPR][RP] (allocated [DK][RP])
    static constexpr int OFF_COL = OFF_RED + DK * RP;     // [DV]
    static constexpr int OFF_W = OFF_COL + DV;            // [C][DV]
    static constexpr int OFF_TOK = OFF_W + C * DV;        // [2][TOK]
    static constexpr int FLOATS = OFF_TOK + 2 * TOK;
    static_assert(NTH % DV == 0 && NPR % TPC == 0 && SW % 4 == 0 && TPC >= 2 && TPC <= 8, "layout");
};

// per (b, h): the NC interval starts, then up to C per-token states
template <int DK, int DV>
size_t ws_bytes(int B, int T, int H) {
    const size_t NC = (size_t)(T + C - 1) / C;
    return (size_t)B * H * (NC + (size_t)min(C, T)) * DK * DV * 4;
}

template <class E, int DK, int DV>
__global__ __launch_bounds__(4 * DK) void recurrent_bwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ z,
    const E* __restrict__ beta, float g_min, const float* __restrict__ s0, const E* __restrict__ dout,
    const float* __restrict__ ds_final, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dz, float* __restrict__ dbeta, float* __restrict__ ds0, int T, int H,
    float* __restrict__ ws) {
    typedef BLay<DK, DV> L;
    constexpr int SW = L::SW;
    extern __shared__ __align__(16) float lds[];
    float* red = lds + L::OFF_RED;
    float* col = lds + L::OFF_COL;
    float* wbuf = lds + L::OFF_W;
    const int tid = threadIdx.x, r = tid >> 2, g = tid & 3, c0 = g * SW;
    const size_t bh = blockIdx.x;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int NC = (T + C - 1) / C;
    float* ckpt = ws + bh * (size_t)(NC + min(C, T)) * DK * DV;   // [NC][DK][DV]
    float* pre = ckpt + (size_t)NC * DK * DV;                     // [min(C, T)][DK][DV]
    const size_t own = (size_t)r * DV + c0;               // this thread's elements of a DK x DV matrix
    auto row_of = [&](int t) { return ((size_t)b * T + t) * H + h; };

    // A token's inputs are fetched into registers (item i of q | k | z |
    // v or do | beta per thread, i = tid + u NTH) one step ahead and put
    // into the staging buffer of its step between the last two barriers of
    // the step before, whose last barrier publishes them: their load latency
    // hides behind that step, and a step needs two barriers (the column-sum
    // partials, then the column sums and the next token).
    constexpr int NIT = 3 * DK + DV + 1;
    constexpr int IPT = (NIT + L::NTH - 1) / L::NTH;
    // The source is selected first and loaded without a branch, and the raw
    // value is converted only when put, so that the load stays in flight
    // until then.
    E fv[IPT];
    auto fetch = [&](int t, bool fwd) {
        const size_t rt = row_of(t);
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int i = min(tid + u * L::NTH, NIT - 1);
            const E* src = i < DK ? q + rt * DK + i
                         : i < 2 * DK ? k + rt * DK + (i - DK)
                         : i < 3 * DK ? z + rt * DK + (i - 2 * DK)
                         : i < 3 * DK + DV ? (fwd ? v : dout) + rt * DV + (i - 3 * DK)
                         : beta + rt;
            fv[u] = *src;
        }
    };
    auto put = [&](float* tb) {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int i = tid + u * L::NTH;
            const float x = to_f32(fv[u]);
            if (i < 2 * DK) {
                tb[i] = x;
            } else if (i < 3 * DK) {
                const int c = i - 2 * DK;
                const float sg = 1.0f / (1.0f + expf(-x));
                const float a = expf(g_min * sg);
                tb[2 * DK + c] = a;
                tb[3 * DK + c] = a * g_min * sg * (1.0f - sg);
            } else if (i < 3 * DK + DV) {
                tb[4 * DK + i - 3 * DK] = x;
            } else if (i < NIT) {
                tb[4 * DK + DV] = x;
            }
        }
    };
    auto tok_buf = [&](int par) { return lds + L::OFF_TOK + par * L::TOK; };
    // Column sums of x[c] (this thread's row, its quarter's columns) over
    // all rows: the four rows held by the lanes of a 16-lane DPP row that
    // share a quarter are summed by two row rotations, lanes 16k + g write
    // partial row (16-lane group) to red, and after the barrier col_sums adds
    // the partial rows.
    auto partial_rows = [&](float (&x)[SW]) {
#pragma unroll
        for (int c = 0; c < SW; ++c) {
            float y = x[c];
            y += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, y), 0x124, 0xF, 0xF, false));
            y += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, y), 0x128, 0xF, 0xF, false));
            x[c] = y;
        }
        if ((tid & 12) == 0) {
            float* pr = red + (tid >> 4) * L::RP + c0;
#pragma unroll
            for (int c = 0; c < SW; c += 4) *reinterpret_cast<f32x4*>(pr + c) = f32x4{x[c], x[c + 1], x[c + 2], x[c + 3]};
        }
    };
    // lane exchanges within a group of four lanes (DPP quad permutes)
    auto xor1 = [](float x) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    };
    auto xor2 = [](float x) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    };
    // col[c] = sum over the partial rows of red[.][c] (taken TPC apart by the threads of a column)
    auto col_sums = [&]() {
        const int cc = tid / L::TPC, jj = tid % L::TPC;
        float acc = 0.f;
#pragma unroll 8
        for (int i = 0; i < L::RPT; ++i) acc += red[(i * L::TPC + jj) * L::RP + cc];
        acc += xor1(acc);
        if constexpr (L::TPC >= 4) acc += xor2(acc);
        if constexpr (L::TPC >= 8) acc += __shfl_xor(acc, 4);
        if (jj == 0) col[cc] = acc;
    };
    auto quad_sum = [&](float x) {
        x += xor1(x);
        x += xor2(x);
        return x;
    };

    float s[SW], ds[SW];
    // one token forward: s <- S_t from S_{t-1}, the token staged (and
    // published) in buffer par; with keep_w, w into wbuf[j].  tn >= 0: the
    // next step's token, fetched here (forward step when fn) and staged in
    // buffer par ^ 1.
    auto fwd_step = [&](int par, bool keep_w, int j, int tn, bool fn) {
        float* tb = tok_buf(par);
        if (tn >= 0) fetch(tn, fn);
        const float a = tb[2 * DK + r], kr = tb[DK + r], bt = tb[4 * DK + DV];
        float x[SW];
#pragma unroll
        for (int c = 0; c < SW; ++c) {
            s[c] *= a;
            x[c] = s[c] * kr;
        }
        partial_rows(x);
        __syncthreads();
        col_sums();
        if (tn >= 0) put(tok_buf(par ^ 1));
        __syncthreads();
#pragma unroll
        for (int c = 0; c < SW; ++c) {
            const float w = tb[4 * DK + c0 + c] - col[c0 + c];
            if (keep_w && r == 0) wbuf[j * DV + c0 + c] = w;
            s[c] += bt * kr * w;
        }
    };

    // ---- forward sweep: the state at the start of every interval
#pragma unroll
    for (int c = 0; c < SW; ++c) s[c] = s0 ? s0[bh * DK * DV + own + c] : 0.f;
    int par = 0;
    if (T > 0) {
        fetch(0, true);
        put(tok_buf(0));
        __syncthreads();
    }
    for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int c = 0; c < SW; c += 4)
            *reinterpret_cast<f32x4*>(ckpt + (size_t)n * DK * DV + own + c) = f32x4{s[c], s[c + 1], s[c + 2], s[c + 3]};
        const int t1 = min(T, (n + 1) * C);
        for (int t = n * C; t < t1; ++t, par ^= 1) fwd_step(par, false, 0, t + 1 < T ? t + 1 : -1, true);
    }

    // ---- backward sweep
#pragma unroll
    for (int c = 0; c < SW; ++c) ds[c] = ds_final ? ds_final[bh * DK * DV + own + c] : 0.f;
    for (int n = NC - 1; n >= 0; --n) {
        const int t0 = n * C, len = min(C, T - t0);
#pragma unroll
        for (int c = 0; c < SW; c += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(ckpt + (size_t)n * DK * DV + own + c);
            s[c] = x[0];
            s[c + 1] = x[1];
            s[c + 2] = x[2];
            s[c + 3] = x[3];
        }
        // the interval forward again: each token's incoming state, and w;
        // its last step fetches the first backward step's token
        __syncthreads();   // the previous step's reads of both staging buffers done
        fetch(t0, true);
        put(tok_buf(par));
        __syncthreads();
        for (int j = 0; j < len; ++j, par ^= 1) {
#pragma unroll
            for (int c = 0; c < SW; c += 4)
                *reinterpret_cast<f32x4*>(pre + (size_t)j * DK * DV + own + c) =
                    f32x4{s[c], s[c + 1], s[c + 2], s[c + 3]};
            const bool last = j + 1 == len;
            fwd_step(par, true, j, last ? t0 + len - 1 : t0 + j + 1, !last);
        }
        // then back through its tokens; s is S_t on entry to each step
        for (int j = len - 1; j >= 0; --j, par ^= 1) {
            const int t = t0 + j;
            const size_t rt = row_of(t);
            float* tb = tok_buf(par);
            float sp[SW];   // S_{t-1}
#pragma unroll
            for (int c = 0; c < SW; c += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(pre + (size_t)j * DK * DV + own + c);
                sp[c] = x[0];
                sp[c + 1] = x[1];
                sp[c + 2] = x[2];
                sp[c + 3] = x[3];
            }
            if (j > 0) fetch(t - 1, false);
            const float a = tb[2 * DK + r], kr = tb[DK + r], qr = tb[r], bt = tb[4 * DK + DV];
            const float* dov = tb + 4 * DK;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < SW; ++c) acc += s[c] * dov[c0 + c];
            acc = quad_sum(acc);
            if (g == 0) dq[rt * DK + r] = acc;
            float x[SW];
#pragma unroll
            for (int c = 0; c < SW; ++c) {
                ds[c] += qr * dov[c0 + c];
                x[c] = ds[c] * kr;
            }
            partial_rows(x);
            __syncthreads();
            col_sums();
            if (j > 0) put(tok_buf(par ^ 1));
            __syncthreads();
            float dbt = 0.f, dkr = 0.f, dal = 0.f;
#pragma unroll
            for (int c = 0; c < SW; ++c) {
                const float u = col[c0 + c], w = wbuf[j * DV + c0 + c];
                const float dw = bt * u;
                dbt += u * w;
                dkr += bt * ds[c] * w - a * sp[c] * dw;
                const float dsp = ds[c] - kr * dw;
                dal += sp[c] * dsp;
                ds[c] = a * dsp;
                if (r == 0) dv[rt * DV + c0 + c] = dw;
                s[c] = sp[c];
            }
            dbt = quad_sum(dbt);
            dkr = quad_sum(dkr);
            dal = quad_sum(dal);
            if (tid == 0) dbeta[rt] = dbt;
            if (g == 0) {
                dk[rt * DK + r] = dkr;
                dz[rt * DK + r] = dal * tb[3 * DK + r];
            }
        }
    }
    if (ds0) {
#pragma unroll
        for (int c = 0; c < SW; c += 4)
            *reinterpret_cast<f32x4*>(ds0 + bh * DK * DV + own + c) = f32x4{ds[c], ds[c + 1], ds[c + 2], ds[c + 3]};
    }
}

template <class E, int DK, int DV>
hipError_t launch_t(const BwdArgs& a) {
    typedef BLay<DK, DV> L;
    const size_t lds = (size_t)L::FLOATS * 4;
    hipError_t err = hipFuncSetAttribute((const void*)recurrent_bwd_kernel<E, DK, DV>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((recurrent_bwd_kernel<E, DK, DV>), dim3(a.B * a.H), dim3(L::NTH), lds,
                       (hipStream_t)a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.z,
                       (const E*)a.beta, a.g_min, a.s0, (const E*)a.dout, a.ds_final, a.dq, a.dk, a.dv, a.dz,
                       a.dbeta, a.ds0, a.T, a.H, (float*)a.workspace);
    return hipGetLastError();
}

template <class E>
hipError_t launch_e(const BwdArgs& a) {
    if (a.dk_dim == 128 && a.dv_dim == 128) return launch_t<E, 128, 128>(a);
    if (a.dk_dim == 128 && a.dv_dim == 64) return launch_t<E, 128, 64>(a);
    if (a.dk_dim == 64 && a.dv_dim == 128) return launch_t<E, 64, 128>(a);
    return launch_t<E, 64, 64>(a);
}

}  // namespace bwdk

size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv) {
    if (dk == 128 && dv == 128) return bwdk::ws_bytes<128, 128>(B, T, H);
    if (dk == 128 && dv == 64) return bwdk::ws_bytes<128, 64>(B, T, H);
    if (dk == 64 && dv == 128) return bwdk::ws_bytes<64, 128>(B, T, H);
    return bwdk::ws_bytes<64, 64>(B, T, H);
}

hipError_t launch_bwd(const BwdArgs& a) {
    return a.bf16 ? bwdk::launch_e<bf16>(a) : bwdk::launch_e<float>(a);
}

}  // namespace kda
