// gemm.hip -- the output projection of the KDA layer ("KDA Recurrence"
// problem statement: heads concatenated to width H*d_v, then out = y W^T with
// W of shape (d_model, H*d_v) and no bias):
//
//   out (M x N, bf16) = A (M x K, bf16) . B (N x K, bf16)^T,  fp32 accumulation.
//
// Both operands are K-contiguous, the native operand layout of the MFMA, so
// tiles go from global memory straight into LDS (global_load_lds_dwordx4,
// no register staging) and from LDS into v_mfma_f32_16x16x32_bf16 operands
// without any transpose.
//
//  * proj_gemm_kernel<BM, BN, NWM, NWN>: a BM x BN output tile per workgroup
//    of NWM x NWN waves, K in 32-deep stages, four LDS stages: a stage is
//    loaded three iterations before it is multiplied and its fragments are
//    read into registers one iteration before, behind the MFMAs of the
//    previous stage.
//  * LDS rows hold 32 bf16 (64 bytes) as four 16-byte groups, swizzled so
//    that the lanes one LDS pass serves in a fragment read hit distinct banks.
//  * Workgroups are dealt round-robin to the 8 XCDs; tile indices are
//    assigned so that consecutive workgroups on one XCD share an A row tile
//    (and walk the B tiles together), which keeps both in that XCD's L2.
//  * Results leave through LDS so that every global store is 16 bytes.
//  * Small M (a decode batch): the K range is split over eight workgroups
//    per tile (proj_gemm_kernel with KSPLIT > 1 writes fp32 partial tiles to
//    the caller's scratch) and split_sum_kernel adds the partials in a fixed
//    order, so the result is deterministic.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace gemmk {

constexpr int BK = 32;            // K per stage
constexpr int NSTAGE = 4;         // LDS stages: three are loading while one is multiplied
constexpr int ROWB = BK * 2;      // bytes per LDS row

// Byte offset of 16-byte group kc (k = 8 kc .. 8 kc + 7) of row `row` in a
// stage.  A 16-byte LDS read of a wave is served 16 lanes at a time, lanes
// 8p .. 8p+7 together with lanes 8p+16 .. 8p+23; in a fragment read those are
// eight consecutive rows at groups kc and kc + 1 (kc even).  Storing group kc
// of row r at kc ^ (2 if r % 8 >= 4) puts those sixteen 16-byte reads on
// sixteen distinct positions of the 256-byte bank space.
__device__ __forceinline__ int swz(int row, int kc) { return row * ROWB + ((kc ^ ((row >> 1) & 2)) << 4); }

// s_waitcnt immediate for vmcnt(N) alone (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
constexpr unsigned vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    return (unsigned)((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

template <int BM, int BN, int NWM, int NWN>
struct Cfg {
    static constexpr int NW = NWM * NWN, NTH = 64 * NW;
    static constexpr int WM = BM / NWM, WN = BN / NWN;     // wave tile
    static constexpr int TM = WM / 16, TN = WN / 16;       // 16x16 MFMA tiles per wave
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LOADS = (BM + BN) / 16 / NW;      // load instructions per wave per stage
    static constexpr int EPITCH = WN * 2 + 16;              // epilogue row pitch (bytes)
    static constexpr int EPI = NW * WM * EPITCH;
    static constexpr int LDS = NSTAGE * STAGE > EPI ? NSTAGE * STAGE : EPI;
    static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "whole load instructions per wave");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
};

// One operand tile (ROWS x 32 bf16 at rows row0.., columns k0..) into LDS:
// wave instruction i fills 1 KB, i.e. rows 16i .. 16i+15; rows past rowmax
// repeat rowmax (always in bounds; those results are never stored).
template <int ROWS, int NW>
__device__ __forceinline__ void load_tile(const bf16* __restrict__ src, int ld, int row0, int rowmax, int k0,
                                          unsigned char* lds) {
    constexpr int PER_WAVE = ROWS / 16 / NW;
    const int w = wave_id(), l = lane_id();
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int ins = w * PER_WAVE + i;
        const int row = ins * 16 + (l >> 2), slot = l & 3;
        const int kc = slot ^ ((row >> 1) & 2);
        const bf16* g = src + (size_t)min(row0 + row, rowmax) * ld + k0 + kc * 8;
        __builtin_amdgcn_global_load_lds(g, lds + ins * 1024, 16, 0, 0);
    }
}

// Tile (tm, tn) and K split sp of workgroup `id`.  Workgroups are dealt to
// the XCDs round-robin (id on XCD id % 8), so the workgroups XCD x receives
// in turn (j = id / 8) take the N tiles of one M tile one after the other:
// that A row tile stays in the XCD's L2 while the B tiles stream past.  M
// tiles beyond the last multiple of 8 are dealt in plain order.
__device__ __forceinline__ void tile_of(int id, int mt, int nt, int& tm, int& tn, int& sp) {
    sp = id / (mt * nt);
    const int r = id % (mt * nt);
    const int full = (mt / 8) * 8;          // M tiles dealt XCD by XCD
    if (r < full * nt) {
        const int x = r & 7, j = r >> 3;
        tm = (j / nt) * 8 + x;
        tn = j % nt;
    } else {
        const int t = r - full * nt;
        tm = full + t / nt;
        tn = t % nt;
    }
}

// out = A . B^T over the K range of split sp (KSPLIT > 1: fp32 partial tile
// into part[sp] instead of bf16 into out).
template <int BM, int BN, int NWM, int NWN, int KSPLIT>
__global__ __launch_bounds__(64 * NWM * NWN) void proj_gemm_kernel(const bf16* __restrict__ A,
                                                                   const bf16* __restrict__ B,
                                                                   bf16* __restrict__ out, float* __restrict__ part,
                                                                   int M, int N, int K) {
    typedef Cfg<BM, BN, NWM, NWN> L;
    extern __shared__ __align__(16) unsigned char smem[];
    const int mt = (M + BM - 1) / BM, nt = N / BN;
    int tm, tn, sp;
    tile_of(blockIdx.x, mt, nt, tm, tn, sp);
    const int m0 = tm * BM, n0 = tn * BN;
    const int w = wave_id(), l = lane_id(), g = l >> 4, cl = l & 15;
    const int wm = w / NWN, wn = w % NWN;
    const int nk_all = K / BK, nk = nk_all / KSPLIT, kt0 = sp * nk;

    f32x4 acc[L::TM][L::TN];
#pragma unroll
    for (int i = 0; i < L::TM; ++i)
#pragma unroll
        for (int j = 0; j < L::TN; ++j) acc[i][j] = zero4();

    auto issue = [&](int kt, int stage) {
        unsigned char* s = smem + stage * L::STAGE;
        load_tile<BM, L::NW>(A, K, m0, M - 1, kt * BK, s);
        load_tile<BN, L::NW>(B, K, n0, N - 1, kt * BK, s + L::A_BYTES);
    };
    // fragments of one stage, read from LDS
    typedef bf16x8 Frags[L::TM + L::TN];
    auto read_frags = [&](Frags& f, int stage) {
        const unsigned char* As = smem + stage * L::STAGE;
        const unsigned char* Bs = As + L::A_BYTES;
#pragma unroll
        for (int i = 0; i < L::TM; ++i) f[i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * L::WM + 16 * i + cl, g));
#pragma unroll
        for (int j = 0; j < L::TN; ++j)
            f[L::TM + j] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * L::WN + 16 * j + cl, g));
    };
    auto multiply = [&](const Frags& f) {
#pragma unroll
        for (int i = 0; i < L::TM; ++i)
#pragma unroll
            for (int j = 0; j < L::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[i], f[L::TM + j], acc[i][j], 0, 0, 0);
    };
    // Stage s is loaded (global -> LDS) three iterations ahead; its
    // fragments are read (LDS -> registers) one iteration ahead, while the
    // previous stage's fragments feed the MFMAs.  Loads past the last stage
    // repeat it (always in bounds, never used).
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s) issue(kt0 + min(s, nk - 1), s);
    __builtin_amdgcn_s_waitcnt(vm_wait<L::LOADS * (NSTAGE - 2)>());   // stage 0 of this wave
    __builtin_amdgcn_s_barrier();                                      // ... and of every wave
    Frags f0, f1;
    read_frags(f0, 0);
    // one iteration: stage `it` multiplied from `cur` while stage it + 1 is
    // read into `nxt` (a plain s_barrier: __syncthreads would also wait for
    // every global load in flight)
    auto step = [&](int it, const Frags& cur, Frags& nxt) {
        __builtin_amdgcn_s_waitcnt(vm_wait<L::LOADS>());   // stage it + 1 landed (it + 2 may not have)
        __builtin_amdgcn_s_waitcnt(0xc07f);                 // lgkmcnt(0): stage it's fragments are in
        __builtin_amdgcn_s_barrier();
        read_frags(nxt, (it + 1) % NSTAGE);
        issue(kt0 + min(it + NSTAGE - 1, nk - 1), (it + NSTAGE - 1) % NSTAGE);
        multiply(cur);
    };
    int it = 0;
    for (; it + 2 <= nk; it += 2) {
        step(it, f0, f1);
        step(it + 1, f1, f0);
    }
    if (it < nk) step(it, f0, f1);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the trailing (unused) stage loads
    __syncthreads();                      // every wave is done with the stages

    if constexpr (KSPLIT > 1) {
        // fp32 partial tile, rows m0.., columns n0.. of split sp
        float* p = part + (size_t)sp * M * N;
#pragma unroll
        for (int i = 0; i < L::TM; ++i)
#pragma unroll
            for (int j = 0; j < L::TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + wm * L::WM + 16 * i + 4 * g + e;
                    if (m < M) p[(size_t)m * N + n0 + wn * L::WN + 16 * j + cl] = acc[i][j][e];
                }
    } else {
        // bf16 tile of each wave into LDS, then 16-byte row stores
        unsigned char* e0 = smem + (size_t)w * L::WM * L::EPITCH;
#pragma unroll
        for (int i = 0; i < L::TM; ++i)
#pragma unroll
            for (int j = 0; j < L::TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<bf16*>(e0 + (16 * i + 4 * g + e) * L::EPITCH + (16 * j + cl) * 2) =
                        (bf16)acc[i][j][e];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int UPR = L::WN / 8;                 // 16-byte units per row
        constexpr int UNITS = L::WM * UPR;
#pragma unroll 4
        for (int u = l; u < UNITS; u += 64) {
            const int r = u / UPR, c = u % UPR;
            const int m = m0 + wm * L::WM + r;
            if (m < M)
                *reinterpret_cast<u32x4*>(out + (size_t)m * N + n0 + wn * L::WN + c * 8) =
                    *reinterpret_cast<const u32x4*>(e0 + r * L::EPITCH + c * 16);
        }
    }
}

// out = sum over the nsplit partial tiles, in split order.
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, bf16* __restrict__ out,
                                                        size_t mn, int nsplit) {
    for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < mn; i += (size_t)gridDim.x * 256 * 4) {
        f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
        for (int k = 1; k < nsplit; ++k) s += *reinterpret_cast<const f32x4*>(part + (size_t)k * mn + i);
        *reinterpret_cast<bf16x4*>(out + i) = bf16x4{(bf16)s[0], (bf16)s[1], (bf16)s[2], (bf16)s[3]};
    }
}

template <int BM, int BN, int NWM, int NWN, int KSPLIT>
static hipError_t launch_t(const bf16* a, const bf16* b, bf16* out, float* part, int M, int N, int K,
                           hipStream_t st) {
    typedef Cfg<BM, BN, NWM, NWN> L;
    auto kern = proj_gemm_kernel<BM, BN, NWM, NWN, KSPLIT>;
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS);
    if (err != hipSuccess) return err;
    const int tiles = ((M + BM - 1) / BM) * (N / BN) * KSPLIT;
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(L::NTH), L::LDS, st, a, b, out, part, M, N, K);
    return hipGetLastError();
}

}  // namespace gemmk

// Shapes: N a multiple of 16 and K a multiple of 64 (d_model % 16 == 0,
// K = H * d_v with d_v in {64, 128}).  Large M: 256 x 256 tiles of 4 x 4
// waves (N a multiple of 256) or 128 x 128 tiles; small M (a decode batch):
// 256 x 128 tiles of 4 x 2 waves with the K range split in eight (N a
// multiple of 128 and K of 256).  Other shapes: 64 x 16 tiles of one wave.
bool gemm_small_m(int M) { return M <= 1024; }

// Small M: a decode batch of up to 256 rows in one 256-row tile of 4 x 2
// waves (up to four tiles for M <= 1024), 128 columns, the K range split in eight (measured at M = 256,
// K = 4096, N = 2304 against 64 x 128 tiles split in four, 128 x 128 split
// in four or eight and 256 x 128 split in sixteen: fewer re-reads of W and y
// through L2 outweigh the larger fp32 partial tiles).
constexpr int SM_BM = 256, SM_BN = 128, SM_KS = 8;
static bool split_k(int M, int N, int K) { return gemm_small_m(M) && N % SM_BN == 0 && (K / gemmk::BK) % SM_KS == 0; }

size_t projection_scratch_bytes(int M, int N, int K) { return split_k(M, N, K) ? (size_t)SM_KS * M * N * 4 : 0; }

hipError_t launch_projection(const void* y, const void* w, void* out, int M, int N, int K, void* scratch,
                             void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (M == 0) return hipSuccess;
    const bf16 *a = (const bf16*)y, *b = (const bf16*)w;
    bf16* o = (bf16*)out;
    if (split_k(M, N, K)) {
        float* part = (float*)scratch;
        hipError_t err = gemmk::launch_t<SM_BM, SM_BN, 4, 2, SM_KS>(a, b, o, part, M, N, K, st);
        if (err != hipSuccess) return err;
        const size_t mn = (size_t)M * N;
        const size_t blocks = (mn / 4 + 255) / 256;
        hipLaunchKernelGGL(gemmk::split_sum_kernel, dim3((unsigned)(blocks < 65535 ? blocks : 65535)), dim3(256), 0,
                           st, (const float*)part, o, mn, SM_KS);
        return hipGetLastError();
    }
    if (!gemm_small_m(M) && N % 256 == 0) return gemmk::launch_t<256, 256, 4, 4, 1>(a, b, o, nullptr, M, N, K, st);
    if (!gemm_small_m(M) && N % 128 == 0) return gemmk::launch_t<128, 128, 2, 2, 1>(a, b, o, nullptr, M, N, K, st);
    return gemmk::launch_t<64, 16, 1, 1, 1>(a, b, o, nullptr, M, N, K, st);
}

}  // namespace kda
