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
//  * the projection out (M x N) = y (M x K) . W (N x K)^T is a plain bf16
//    GEMM with fp32 accumulation: it runs on hipBLASLt (one library handle per
//    device, one heuristic query per shape, both cached), with a library
//    workspace appended to the y buffer.  When the library offers no
//    algorithm for a shape, proj_gemm_kernel below computes it.
//  * proj_gemm_kernel: out (M x N) = y (M x K) . W (N x K)^T in bf16 with
//    fp32 accumulation on v_mfma_f32_16x16x32_bf16.  Both operands are
//    K-contiguous, which is the native operand layout of the MFMA, so tiles
//    go global -> registers -> LDS without any transpose.  128x128 block
//    tile, 64-deep K stages, double-buffered LDS, 4 waves of 64x64.
#include <hipblaslt/hipblaslt.h>

#include <mutex>
#include <deque>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

template <class E, int DV>
__global__ __launch_bounds__(256) void gate_kernel(const E* __restrict__ o, const E* __restrict__ gate,
                                                   float eps, E* __restrict__ y, size_t rows) {
    constexpr int LPR = DV / 8;              // lanes per row, 8 values per lane
    constexpr int RPB = 256 / LPR;           // rows per block per iteration
    const int tid = threadIdx.x;
    const int sub = tid % LPR;
    for (size_t row = (size_t)blockIdx.x * RPB + tid / LPR; row < rows; row += (size_t)gridDim.x * RPB) {
        const size_t base = row * DV + sub * 8;
        float x[8], g[8];
        if constexpr (sizeof(E) == 2) {
            const bf16x8 xv = *reinterpret_cast<const bf16x8*>(o + base);
            const bf16x8 gv = *reinterpret_cast<const bf16x8*>(gate + base);
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
            *reinterpret_cast<bf16x8*>(y + base) = out;
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
}

// ---------------------------------------------------------------------------
// Projection GEMM: out[m][n] = sum_k y[m][k] * w[n][k]
// ---------------------------------------------------------------------------
constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;

__device__ __forceinline__ void gemm_gload(u32x4 (&ra)[4], u32x4 (&rb)[4], const bf16* __restrict__ A,
                                           const bf16* __restrict__ Bw, int M, int N, int K, int m0, int n0,
                                           int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int v = threadIdx.x + i * 256, r = v >> 3, cv = v & 7;
        const int am = min(m0 + r, M - 1), bn = min(n0 + r, N - 1);
        ra[i] = *reinterpret_cast<const u32x4*>(A + (size_t)am * K + k0 + cv * 8);
        rb[i] = *reinterpret_cast<const u32x4*>(Bw + (size_t)bn * K + k0 + cv * 8);
    }
}

__device__ __forceinline__ void gemm_sstore(const u32x4 (&ra)[4], const u32x4 (&rb)[4], bf16* As, bf16* Bs) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int v = threadIdx.x + i * 256, r = v >> 3, cv = v & 7;
        *reinterpret_cast<u32x4*>(&As[r * GLD + cv * 8]) = ra[i];
        *reinterpret_cast<u32x4*>(&Bs[r * GLD + cv * 8]) = rb[i];
    }
}

__global__ __launch_bounds__(256) void proj_gemm_kernel(const bf16* __restrict__ A, const bf16* __restrict__ Bw,
                                                        bf16* __restrict__ out, int M, int N, int K) {
    __shared__ __align__(16) bf16 As[2][GBM * GLD];
    __shared__ __align__(16) bf16 Bs[2][GBN * GLD];
    const int tid = threadIdx.x, w = wave_id();
    const int wm = w >> 1, wn = w & 1;                  // 2 x 2 waves of 64 x 64
    const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * GBN;

    u32x4 ra[4], rb[4];   // global -> register staging, 4 x 8 bf16 per operand per thread

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

    const int nk = K / GBK;
    gemm_gload(ra, rb, A, Bw, M, N, K, m0, n0, 0);
    gemm_sstore(ra, rb, As[0], Bs[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gemm_gload(ra, rb, A, Bw, M, N, K, m0, n0, (kt + 1) * GBK);
#pragma unroll
        for (int ks = 0; ks < GBK; ks += 32) {
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = load_frag<bf16>(As[buf], GLD, wm * 64 + i * 16, ks);
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = load_frag<bf16>(Bs[buf], GLD, wn * 64 + j * 16, ks);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = Mfma<bf16>::mma(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < nk) gemm_sstore(ra, rb, As[buf ^ 1], Bs[buf ^ 1]);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * 64 + i * 16 + acc_row(e);
                const int n = n0 + wn * 64 + j * 16 + acc_col();
                if (m < M && n < N) out[(size_t)m * N + n] = (bf16)acc[i][j][e];
            }
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

// Library workspace for the projection GEMM, after the y buffer.
constexpr size_t LT_WS = (size_t)32 << 20;

static size_t y_bytes(int B, int T, int H, int dv) { return ((size_t)B * T * H * dv * 2 + 255) / 256 * 256; }

size_t gate_workspace_bytes(int B, int T, int H, int dv, int d_model, bool bf16, bool proj) {
    (void)d_model; (void)bf16;
    if (!proj) return 0;
    return y_bytes(B, T, H, dv) + LT_WS;   // gated activations y (bf16), then the GEMM's workspace
}

namespace {
// One hipBLASLt handle per device and the chosen algorithm per (device, M,
// N, K), created on first use.  Column-major view: out^T (N x M) =
// W (stored K x N, transposed) . y^T (stored K x M).
struct LtPlan {
    int dev, M, N, K;
    bool ok;
    hipblasLtMatmulDesc_t op;
    hipblasLtMatrixLayout_t a, b, c;
    hipblasLtMatmulAlgo_t algo;
    size_t ws;
};
struct LtState {
    std::mutex mu;
    hipblasLtHandle_t handle[64] = {};
    std::deque<LtPlan> plans;   // push_back keeps references to earlier plans valid
};
LtState& lt_state() {
    static LtState s;
    return s;
}

const LtPlan* lt_plan(int dev, int M, int N, int K) {
    LtState& s = lt_state();
    std::lock_guard<std::mutex> lock(s.mu);
    for (const LtPlan& p : s.plans)
        if (p.dev == dev && p.M == M && p.N == N && p.K == K) return p.ok ? &p : nullptr;
    LtPlan p{dev, M, N, K, false, nullptr, nullptr, nullptr, nullptr, {}, 0};
    if (dev < 0 || dev >= 64) return nullptr;
    if (!s.handle[dev] && hipblasLtCreate(&s.handle[dev]) != HIPBLAS_STATUS_SUCCESS) s.handle[dev] = nullptr;
    hipblasLtHandle_t h = s.handle[dev];
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    const uint64_t wsmax = LT_WS;
    hipblasLtMatmulPreference_t pref = nullptr;
    hipblasLtMatmulHeuristicResult_t res{};
    int count = 0;
    bool ok = h && hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.c, HIP_R_16BF, N, M, N) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                                    sizeof(wsmax)) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulAlgoGetHeuristic(h, p.op, p.a, p.b, p.c, p.c, pref, 1, &res, &count) ==
                  HIPBLAS_STATUS_SUCCESS &&
              count > 0 && res.workspaceSize <= LT_WS;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (ok) {
        p.algo = res.algo;
        p.ws = res.workspaceSize;
    }
    p.ok = ok;
    s.plans.push_back(p);
    return ok ? &s.plans.back() : nullptr;
}
}  // namespace

size_t projection_scratch_bytes() { return LT_WS; }

hipError_t launch_projection(const void* y, const void* w, void* out, int M, int N, int K, void* lt_ws,
                             void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (M == 0) return hipSuccess;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (const LtPlan* p = lt_plan(dev, M, N, K)) {
        const float one = 1.f, zero = 0.f;
        const hipblasStatus_t r = hipblasLtMatmul(lt_state().handle[dev], p->op, &one, w, p->a, y, p->b, &zero, out,
                                                  p->c, out, p->c, &p->algo, lt_ws, p->ws, st);
        return r == HIPBLAS_STATUS_SUCCESS ? hipGetLastError() : hipErrorLaunchFailure;
    }
    dim3 grid((N + GBN - 1) / GBN, (M + GBM - 1) / GBM);
    hipLaunchKernelGGL(proj_gemm_kernel, grid, dim3(256), 0, st, (const bf16*)y, (const bf16*)w, (bf16*)out, M, N,
                       K);
    return hipGetLastError();
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
