// chunk.hip -- kda_chunk_fwd: chunkwise KDA prefill on gfx950.
//
// The chunk form (Kimi Linear tech report, section 3.1 and appendix B,
// Propositions 1-2, Eqs. 16-19, with beta_r scaling the whole right-hand
// side of Eqs. 17 and 19).  Inside one 64-token chunk with entering state S:
//   g_r   = g_min * sigmoid(z_r)             (per key channel)
//   G_r   = sum_{j<=r} g_j                   (chunk-local, so e^{G_r} = gamma_r)
//   A_ri  = beta_r sum_c k_rc k_ic e^{G_rc - G_ic}     i < r   (0 otherwise)
//   M_ri  =        sum_c q_rc k_ic e^{G_rc - G_ic}     i <= r  (0 otherwise)
//   (I + A) W = diag(beta) (K * e^G),  (I + A) U = diag(beta) V
//   V_new = U - W S                       (the w/u recurrences in matrix form)
//   O     = (Q * e^G) S + M V_new          (o_r = S_r^T q_r, Eqs. 16 + 18)
//   S'    = Diag(e^{G_C}) S + (K * e^{G_C - G})^T V_new
// The unit-lower system I + A is solved by blocked forward substitution on
// 16x16 blocks, giving the lower-triangular T = (I + A)^{-1}; W = T R_K and
// U = T R_V are then MFMA products.
//
// Two kernels:
//  * chunk_intra_kernel, one workgroup per (chunk, head, batch): everything
//    that depends only on the chunk's own tokens (gate, decay scan, A, M,
//    the solve, W, U, Q*e^G, K*e^{G_C-G}, e^{G_C}), written to the
//    workspace.  Fully parallel over chunks.
//  * chunk_inter_kernel, one workgroup per (value-column tile, head, batch):
//    the sequential chunk-to-chunk recurrence.  The columns of S evolve
//    independently (the transition multiplies S only from the left), so the
//    d_v columns are split into tiles of TV to put more chains on the chip.
//    The fp32 state tile lives in MFMA accumulators for the whole sequence;
//    each wave loads its MFMA operands for the next chunk straight from
//    global memory into registers while the current chunk is computed, and
//    only S^T and V_new^T, which every wave needs, go through LDS.
//
// Overflow: e^{G_r - G_i} is never formed as e^{G_r} e^{-G_i} over the whole
// chunk (|G| reaches 64 * |g_min|, far beyond the fp32 range).  A and M are
// evaluated per 16x16 block (R, I) with reference rows m(R) = 16R + 7:
//   e^{G_r - G_i} = e^{G_r - G_m(R)} * e^{G_m(R) - G_m(I)} * e^{G_m(I) - G_i}.
// The outer factors have exponents bounded by 8 |g_min|; the middle one is
// <= 1 (it underflows to 0 only when the exact product is negligible).
#include "kda_device.hpp"
#include "kda_internal.hpp"

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

// ---------------------------------------------------------------------------
// Intra-chunk work of one (b, h, chunk): 256 threads.
// ---------------------------------------------------------------------------
template <class E, int DK, int DV>
struct Intra {
    typedef typename Compute<E>::type CT;
    static constexpr int NPART = 256 / DK;   // threads per key channel
    static constexpr int RP = C / NPART;     // rows per thread (16 or 32)
    static constexpr int NPV = 256 / DV;
    static constexpr int RPV = C / NPV;
    static constexpr int LDK = DK + 8;       // K-contiguous tile stride (CT)
    static constexpr int LC = C + 8;         // token-contiguous tile stride (CT)
    static constexpr int LA = C + 4;         // fp32 64x64 tile strides
    static constexpr int LT = C + 4;
    static constexpr size_t TILE = (size_t)C * LDK * sizeof(CT);
    // region 1: KL, QL, KR during phases 1-3; then As, Ts, Xs and R_V^T
    static constexpr size_t OFF_RV = (size_t)C * LA * 4 + (size_t)C * LT * 4 + 3 * SUB * SUB * 4;
    static constexpr size_t R1 = align16(cmax(3 * TILE, OFF_RV + (size_t)DV * LC * sizeof(CT)));
    static constexpr size_t OFF_RT = R1;     // R_K^T [DK][LC]
    static constexpr size_t OFF_DSC = OFF_RT + align16((size_t)DK * LC * sizeof(CT));
    static constexpr size_t OFF_GM = OFF_DSC + 6 * DK * 4;
    static constexpr size_t OFF_CAR = OFF_GM + 5 * DK * 4;
    static constexpr size_t OFF_BET = OFF_CAR + NPART * DK * 4;
    static constexpr size_t LDS = OFF_BET + C * 4;
    static_assert(RP % 16 == 0 && RPV % 8 == 0, "intra tiling");
};

// Block pairs (R, I), I <= R, of A and M handled by each of the 4 waves.
__constant__ int kPairs[4][3][2] = {{{0, 0}, {1, 0}, {3, 3}},
                                    {{1, 1}, {2, 0}, {3, 2}},
                                    {{2, 1}, {2, 2}, {3, 1}},
                                    {{3, 0}, {-1, -1}, {-1, -1}}};

template <class E, int DK, int DV>
__device__ __forceinline__ void intra_chunk(const E* __restrict__ q, const E* __restrict__ k,
                                            const E* __restrict__ v, const E* __restrict__ z,
                                            const E* __restrict__ beta, float g_min, int valid, size_t row0,
                                            int H, unsigned char* __restrict__ blk, unsigned char* smem) {
    typedef Intra<E, DK, DV> L;
    typedef typename L::CT CT;
    typedef Mfma<CT> MF;
    typedef Ws<CT, DK, DV> WL;
    constexpr int LDK = L::LDK, LC = L::LC, LA = L::LA, LT = L::LT, RP = L::RP, RPV = L::RPV;

    CT* KL = reinterpret_cast<CT*>(smem);             // [C][LDK] k * e^{G_r - G_m(R)}
    CT* QL = KL + C * LDK;                              // [C][LDK] q * e^{G_r - G_m(R)}
    CT* KR = QL + C * LDK;                              // [C][LDK] k * e^{G_m(R) - G_r}
    float* As = reinterpret_cast<float*>(smem);         // [C][LA]   (after phase 3)
    float* Ts = As + C * LA;                            // [C][LT]
    float* Xs = Ts + C * LT;                            // [3][16][16]
    CT* RT = reinterpret_cast<CT*>(smem + L::OFF_RT);   // [DK][LC] R_K^T = (beta k e^G)^T
    CT* RV = reinterpret_cast<CT*>(smem + L::OFF_RV);   // [DV][LC] R_V^T = (beta v)^T (after phase 3)
    float* dsc = reinterpret_cast<float*>(smem + L::OFF_DSC);   // [6][DK] e^{G_m(R) - G_m(I)}
    float* gm = reinterpret_cast<float*>(smem + L::OFF_GM);     // [5][DK] G_m(R), G_C
    float* car = reinterpret_cast<float*>(smem + L::OFF_CAR);   // [NPART][DK]
    float* bet = reinterpret_cast<float*>(smem + L::OFF_BET);   // [C]

    CT* gW = reinterpret_cast<CT*>(blk) + WL::W;
    CT* gUT = reinterpret_cast<CT*>(blk) + WL::UT;
    CT* gM = reinterpret_cast<CT*>(blk) + WL::M;
    CT* gQG = reinterpret_cast<CT*>(blk) + WL::QG;
    CT* gKGT = reinterpret_cast<CT*>(blk) + WL::KGT;
    float* gEGC = reinterpret_cast<float*>(reinterpret_cast<CT*>(blk) + WL::END);

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();

    // ---- phase 1: gate and chunk-local scan, one key channel per thread group
    if (tid < C) bet[tid] = tid < valid ? to_f32(beta[row0 + (size_t)tid * H]) : 0.f;
    const int c = tid % DK, part = tid / DK, r0 = part * RP;
    const int cv = tid % DV, rv0 = (tid / DV) * RPV;
    // All global loads first, at clamped (always valid) rows and without any
    // branch, so they are in flight together; rows past the end of the
    // sequence are then zeroed arithmetically.
    E zr[RP], kr[RP], qr[RP], vr[RPV];
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const size_t off = (row0 + (size_t)min(r0 + i, valid - 1) * H) * DK + c;
        zr[i] = z[off];
        kr[i] = k[off];
        qr[i] = q[off];
    }
#pragma unroll
    for (int i = 0; i < RPV; ++i) vr[i] = v[(row0 + (size_t)min(rv0 + i, valid - 1) * H) * DV + cv];
    float G[RP], kv[RP], qv[RP], vv[RPV];
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const float msk = r0 + i < valid ? 1.f : 0.f;
        G[i] = msk * (g_min * dsigmoid<E>(to_f32(zr[i])));
        kv[i] = msk * to_f32(kr[i]);
        qv[i] = msk * to_f32(qr[i]);
    }
#pragma unroll
    for (int i = 0; i < RPV; ++i) vv[i] = to_f32(vr[i]);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) { s += G[i]; G[i] = s; }
    car[part * DK + c] = s;
    __syncthreads();
    float carry = 0.f, gC = 0.f;
#pragma unroll
    for (int p = 0; p < L::NPART; ++p) {
        const float t = car[p * DK + c];
        if (p < part) carry += t;
        gC += t;     // same summation order as carry + s of the last part
    }
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        G[i] += carry;
        if ((i & 15) == 7) gm[((r0 + i) >> 4) * DK + c] = G[i];
    }
    if (part == 0) {
        gm[4 * DK + c] = gC;
        gEGC[c] = dexp<E>(gC);
    }
    __syncthreads();

    // ---- phase 2: decay-scaled operands
    {
        constexpr int NB = RP / 16;
        float gmR[NB], eGm[NB], eCGm[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            gmR[j] = gm[((r0 >> 4) + j) * DK + c];
            eGm[j] = dexp<E>(gmR[j]);
            eCGm[j] = dexp<E>(gC - gmR[j]);
        }
        float rk[RP], kg[RP];
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i, j = i >> 4;
            const float el = G[i] - gmR[j];
            const float left = dexp<E>(el), right = dexp<E>(-el);
            const float kL = kv[i] * left, qL = qv[i] * left, kR = kv[i] * right;
            KL[r * LDK + c] = from_f32<CT>(kL);
            QL[r * LDK + c] = from_f32<CT>(qL);
            KR[r * LDK + c] = from_f32<CT>(kR);
            gQG[r * DK + c] = from_f32<CT>(qL * eGm[j]);
            rk[i] = bet[r] * kL * eGm[j];
            kg[i] = kR * eCGm[j];
        }
#pragma unroll
        for (int i = 0; i < RP; i += 8) {
            store8<CT>(RT + c * LC + r0 + i, &rk[i]);
            store8<CT>(gKGT + c * C + r0 + i, &kg[i]);
        }
    }
    for (int idx = tid; idx < 6 * DK; idx += 256) {
        const int p = idx / DK, cc = idx % DK;
        const int R = p < 1 ? 1 : (p < 3 ? 2 : 3);
        const int I = p - R * (R - 1) / 2;
        dsc[idx] = dexp<E>(gm[R * DK + cc] - gm[I * DK + cc]);
    }
    __syncthreads();

    // ---- phase 3: A and M per 16x16 block pair, computed transposed
    //      (D[i][r] = sum_c k'_ic k_rc) so that each lane ends up holding four
    //      consecutive key indices of one row: contiguous row-major stores.
    float av[3][4];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int R = kPairs[w][j][0], I = kPairs[w][j][1];
        if (R < 0) break;
        f32x4 accA = zero4(), accM = zero4();
        const float* dv = dsc + (R * (R - 1) / 2 + I) * DK;
        for (int kk = 0; kk < DK; kk += MF::KSTEP) {
            typename MF::frag ak = load_frag<CT>(KR, LDK, I * SUB, kk);
            if (I < R) {
                float t[MF::KPL];
                MF::to_floats(ak, t);
                const int c0 = kk + (l >> 4) * MF::KPL;
#pragma unroll
                for (int jj = 0; jj < MF::KPL; ++jj) t[jj] *= dv[c0 + jj];
                ak = MF::from_floats(t);
            }
            accA = MF::mma(ak, load_frag<CT>(KL, LDK, R * SUB, kk), accA);
            accM = MF::mma(ak, load_frag<CT>(QL, LDK, R * SUB, kk), accM);
        }
        const int r = R * SUB + (l & 15);
        const int i0 = I * SUB + 4 * (l >> 4);
        f32x4 mv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            av[j][e] = (i0 + e < r) ? bet[r] * accA[e] : 0.f;
            mv[e] = (i0 + e <= r) ? accM[e] : 0.f;
        }
        store4<CT>(gM + r * C + i0, mv);
    }
    if (w == 3) {
        // strictly upper blocks of M are zero
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            const int R = p < 3 ? 0 : (p < 5 ? 1 : 2);
            const int I = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
            store4<CT>(gM + (R * SUB + (l & 15)) * C + I * SUB + 4 * (l >> 4), zero4());
        }
    }
    __syncthreads();   // KL / QL / KR are dead from here on; As, Ts and R_V^T alias them
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int R = kPairs[w][j][0], I = kPairs[w][j][1];
        if (R < 0) break;
        *reinterpret_cast<f32x4*>(As + (R * SUB + (l & 15)) * LA + I * SUB + 4 * (l >> 4)) =
            f32x4{av[j][0], av[j][1], av[j][2], av[j][3]};
    }
#pragma unroll
    for (int i = 0; i < RPV; ++i) vv[i] *= bet[rv0 + i];   // bet is 0 past the end
#pragma unroll
    for (int i = 0; i < RPV; i += 8) store8<CT>(RV + cv * LC + rv0 + i, &vv[i]);
    __syncthreads();

    // ---- phase 4: T = (I + A)^{-1}, blocked forward substitution
    // 4a: diagonal blocks; wave w inverts I + A_ww column by column (lane = column).
    if (l < SUB) {
        const int base = w * SUB;
        float x[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
            float acc = (r == l) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= As[(base + r) * LA + base + i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < SUB; ++r) Ts[(base + r) * LT + base + l] = x[r];
    } else {
        // the other lanes clear the blocks right of the diagonal block
        const int ncols = C - (w + 1) * SUB;
        for (int i = l - SUB; i < SUB * ncols; i += 64 - SUB)
            Ts[(w * SUB + i / ncols) * LT + (w + 1) * SUB + i % ncols] = 0.f;
    }
    __syncthreads();
    // 4b: off-diagonal blocks, one block row at a time:
    //     T_RI = -T_RR * sum_{J=I}^{R-1} A_RJ T_JI
    for (int R = 1; R < 4; ++R) {
        const int rl = tid >> 4, il = tid & 15;
        for (int I = 0; I < R; ++I) {
            float acc = 0.f;
            for (int J = I; J < R; ++J)
#pragma unroll
                for (int t = 0; t < SUB; ++t)
                    acc += As[(R * SUB + rl) * LA + J * SUB + t] * Ts[(J * SUB + t) * LT + I * SUB + il];
            Xs[(I * SUB + rl) * SUB + il] = acc;
        }
        __syncthreads();
        for (int I = 0; I < R; ++I) {
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < SUB; ++t) acc -= Ts[(R * SUB + rl) * LT + R * SUB + t] * Xs[(I * SUB + t) * SUB + il];
            Ts[(R * SUB + rl) * LT + I * SUB + il] = acc;
        }
        __syncthreads();
    }

    // ---- phase 5: W = T R_K (computed as W^T = R_K^T T^T) and U = T R_V;
    //      wave w owns token rows 16w..16w+15 of both.
    {
        constexpr int NKS = C / MF::KSTEP;
        const int ns = (SUB * (w + 1) + MF::KSTEP - 1) / MF::KSTEP;   // T_w. vanishes beyond
        typename MF::frag tf[NKS];
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2)
            tf[s2] = s2 < ns ? load_frag_f32<CT>(Ts, LT, w * SUB, s2 * MF::KSTEP) : typename MF::frag{};
#pragma unroll 2
        for (int cb = 0; cb < DK / 16; ++cb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s2 = 0; s2 < NKS; ++s2)
                if (s2 < ns) acc = MF::mma(load_frag<CT>(RT, LC, cb * 16, s2 * MF::KSTEP), tf[s2], acc);
            store4<CT>(gW + (w * SUB + (l & 15)) * DK + cb * 16 + 4 * (l >> 4), acc);
        }
#pragma unroll 2
        for (int cb = 0; cb < DV / 16; ++cb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s2 = 0; s2 < NKS; ++s2)
                if (s2 < ns) acc = MF::mma(tf[s2], load_frag<CT>(RV, LC, cb * 16, s2 * MF::KSTEP), acc);
            store4<CT>(gUT + (cb * 16 + (l & 15)) * C + w * SUB + 4 * (l >> 4), acc);
        }
    }
}

template <class E, int DK, int DV>
__global__ __launch_bounds__(256) void chunk_intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const E* __restrict__ beta, float g_min, int T, int H, int NC,
    unsigned char* __restrict__ ws) {
    typedef typename Compute<E>::type CT;
    extern __shared__ __align__(16) unsigned char smem[];
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t0 = n * C;
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    unsigned char* blk = ws + (((size_t)b * H + h) * NC + n) * Ws<CT, DK, DV>::BYTES;
    intra_chunk<E, DK, DV>(q, k, v, z, beta, g_min, min(C, T - t0), row0, H, blk, smem);
}

// ---------------------------------------------------------------------------
// Inter-chunk recurrence of one (b, h, value-column tile): 256 threads.
// ---------------------------------------------------------------------------
template <class E, int DK, int DV, int TV>
struct Inter {
    typedef typename Compute<E>::type CT;
    typedef Mfma<CT> MF;
    static constexpr int KS = MF::KSTEP;
    static constexpr int NKD = DK / KS;     // k-steps over d_k
    static constexpr int NKC = C / KS;      // k-steps over the chunk's tokens
    static constexpr int RB = DK / 64;      // 16-row state blocks per wave
    static constexpr int NT = TV / 16;      // 16-column tiles
    static constexpr int LDK = DK + 8, LC = C + 8;
    static constexpr size_t SB_BYTES = (size_t)TV * LDK * sizeof(CT);
    static constexpr size_t LDS = 2 * SB_BYTES + (size_t)TV * LC * sizeof(CT);

    // One chunk's operands as held by one wave (rows 16w.. of W, Q*e^G, M;
    // state rows w*DK/4.. of (K*e^{G_C-G})^T; V_new init; e^{G_C}).
    struct Regs {
        typename MF::frag w[NKD], qg[NKD], m[NKC], kg[RB][NKC];
        typename Raw4<CT>::type u[NT];
        f32x4 eg[RB];
    };

    static __device__ __forceinline__ void load(Regs& r, const unsigned char* blk, int w, int l, int col0) {
        typedef Ws<CT, DK, DV> WL;
        const CT* base = reinterpret_cast<const CT*>(blk);
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) {
            r.w[kk] = load_frag<CT>(base + WL::W, DK, w * 16, kk * KS);
            r.qg[kk] = load_frag<CT>(base + WL::QG, DK, w * 16, kk * KS);
        }
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) {
            r.m[kk] = load_frag<CT>(base + WL::M, C, w * 16, kk * KS);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                r.kg[rb][kk] = load_frag<CT>(base + WL::KGT, C, w * (DK / 4) + rb * 16, kk * KS);
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
            r.u[ct] = load_raw4<CT>(base + WL::UT + (size_t)(col0 + ct * 16 + (l & 15)) * C + w * 16 + 4 * (l >> 4));
        const float* eg = reinterpret_cast<const float*>(base + WL::END);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            r.eg[rb] = *reinterpret_cast<const f32x4*>(eg + w * (DK / 4) + rb * 16 + 4 * (l >> 4));
    }
};

template <class E, int DK, int DV, int TV>
__global__ __launch_bounds__(256) void chunk_inter_kernel(
    E* __restrict__ o, const float* __restrict__ s0, float* __restrict__ s_final, int T, int H,
    int NC, const unsigned char* __restrict__ ws) {
    typedef Inter<E, DK, DV, TV> L;
    typedef typename L::CT CT;
    typedef typename L::MF MF;
    typedef Ws<CT, DK, DV> WL;
    constexpr int LDK = L::LDK, LC = L::LC, RB = L::RB, NT = L::NT, KS = L::KS;

    extern __shared__ __align__(16) unsigned char smem[];
    CT* Sb0 = reinterpret_cast<CT*>(smem);                          // [TV][LDK] S^T, ping
    CT* Sb1 = reinterpret_cast<CT*>(smem + L::SB_BYTES);            // pong
    CT* Vn = reinterpret_cast<CT*>(smem + 2 * L::SB_BYTES);         // [TV][LC] V_new^T

    // 1-D grid of (tile, chain) with the tile index major: workgroups are
    // dealt round-robin to the 8 XCDs, so when the number of chains B*H is a
    // multiple of 8 all value tiles of a chain run on one XCD and read the
    // chain's workspace through the same L2.
    const int nchain = gridDim.x / (DV / TV);
    const int tile = blockIdx.x / nchain;
    const size_t bh = blockIdx.x % nchain;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int l = lane_id(), w = wave_id();
    const int col0 = tile * TV;
    const unsigned char* chain = ws + bh * NC * WL::BYTES;

    // state rows of this lane: w*DK/4 + rb*16 + 4*(l/16) + e ; column ct*16 + l%16
    f32x4 accS[RB][NT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int row = w * (DK / 4) + rb * 16 + 4 * (l >> 4);
            const int col = ct * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                accS[rb][ct][e] = s0 ? s0[(bh * DK + row + e) * DV + col0 + col] : 0.f;
            store4<CT>(Sb0 + col * LDK + row, accS[rb][ct]);
        }

    typename L::Regs cur, nxt;
    L::load(cur, chain, w, l, col0);
    __syncthreads();

    for (int n = 0; n < NC; ++n) {
        CT* sb = (n & 1) ? Sb1 : Sb0;
        CT* sbn = (n & 1) ? Sb0 : Sb1;
        // Unconditional (clamped) prefetch of the next chunk: under a branch the
        // wait-count insertion would assume the no-load path and stall on it.
        L::load(nxt, chain + (size_t)min(n + 1, NC - 1) * WL::BYTES, w, l, col0);

        // V_new = U - W S (rows 16w.. x TV) and O^T = S^T (Q e^G)^T (TV x rows 16w..)
        f32x4 accP[NT], accO[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) { accP[ct] = zero4(); accO[ct] = zero4(); }
#pragma unroll
        for (int kk = 0; kk < L::NKD; ++kk)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const typename MF::frag fs = load_frag<CT>(sb, LDK, ct * 16, kk * KS);
                accP[ct] = MF::mma(cur.w[kk], fs, accP[ct]);
                accO[ct] = MF::mma(fs, cur.qg[kk], accO[ct]);
            }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
            store4<CT>(Vn + (ct * 16 + (l & 15)) * LC + w * 16 + 4 * (l >> 4), widen4(cur.u[ct]) - accP[ct]);
        __syncthreads();

        // O^T += V_new^T M^T ;  S <- Diag(e^{G_C}) S + (K e^{G_C-G})^T V_new
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) accS[rb][ct] *= cur.eg[rb];
#pragma unroll
        for (int kk = 0; kk < L::NKC; ++kk)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const typename MF::frag fv = load_frag<CT>(Vn, LC, ct * 16, kk * KS);
                accO[ct] = MF::mma(fv, cur.m[kk], accO[ct]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) accS[rb][ct] = MF::mma(cur.kg[rb][kk], fv, accS[rb][ct]);
            }
        const int t = n * C + w * 16 + (l & 15);
        if (t < T) {
            E* orow = o + (((size_t)b * T + t) * H + h) * DV + col0;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) store4<E>(orow + ct * 16 + 4 * (l >> 4), accO[ct]);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                store4<CT>(sbn + (ct * 16 + (l & 15)) * LDK + w * (DK / 4) + rb * 16 + 4 * (l >> 4), accS[rb][ct]);
        __syncthreads();
        cur = nxt;
    }

    if (s_final) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const int row = w * (DK / 4) + rb * 16 + 4 * (l >> 4);
                const int col = ct * 16 + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) s_final[(bh * DK + row + e) * DV + col0 + col] = accS[rb][ct][e];
            }
    }
}

// State pass-through for T == 0: s_final = s0 (or zeros).
__global__ void state_copy_kernel(const float* __restrict__ s0, float* __restrict__ s_final, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        s_final[i] = s0 ? s0[i] : 0.f;
}

// ---------------------------------------------------------------------------
template <class E, int DK, int DV>
static hipError_t launch_chunk_t(const ChunkArgs& a) {
    typedef typename Compute<E>::type CT;
    constexpr int TV = sizeof(CT) == 2 ? 32 : 16;
    const int NC = (a.T + C - 1) / C;
    hipStream_t st = (hipStream_t)a.stream;
    typedef Intra<E, DK, DV> LI;
    typedef Inter<E, DK, DV, TV> LX;
    static_assert(LI::LDS <= 160 * 1024, "intra LDS budget");
    static_assert(LX::LDS <= 64 * 1024, "inter LDS budget");
    hipError_t err = hipFuncSetAttribute((const void*)chunk_intra_kernel<E, DK, DV>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)LI::LDS);
    if (err != hipSuccess) return err;
    unsigned char* ws = (unsigned char*)a.workspace;
    hipLaunchKernelGGL((chunk_intra_kernel<E, DK, DV>), dim3(NC, a.H, a.B), dim3(256), LI::LDS, st,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta,
                       a.g_min, a.T, a.H, NC, ws);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((chunk_inter_kernel<E, DK, DV, TV>), dim3((DV / TV) * a.H * a.B), dim3(256), LX::LDS, st,
                       (E*)a.o, a.s0, a.s_final, a.T, a.H, NC, (const unsigned char*)ws);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_chunk_e(const ChunkArgs& a) {
    if (a.dk == 128 && a.dv == 128) return launch_chunk_t<E, 128, 128>(a);
    if (a.dk == 128 && a.dv == 64) return launch_chunk_t<E, 128, 64>(a);
    if (a.dk == 64 && a.dv == 128) return launch_chunk_t<E, 64, 128>(a);
    return launch_chunk_t<E, 64, 64>(a);
}

template <class E>
static size_t ws_bytes_e(int dk, int dv) {
    typedef typename Compute<E>::type CT;
    if (dk == 128 && dv == 128) return Ws<CT, 128, 128>::BYTES;
    if (dk == 128 && dv == 64) return Ws<CT, 128, 64>::BYTES;
    if (dk == 64 && dv == 128) return Ws<CT, 64, 128>::BYTES;
    return Ws<CT, 64, 64>::BYTES;
}

size_t chunk_workspace_bytes(int B, int T, int H, int dk, int dv, bool bf16) {
    const size_t NC = ((size_t)T + C - 1) / C;
    const size_t per = bf16 ? ws_bytes_e<kda::bf16>(dk, dv) : ws_bytes_e<float>(dk, dv);
    return (size_t)B * H * NC * per;
}

hipError_t launch_chunk(const ChunkArgs& a) {
    if (a.T == 0) {
        if (!a.s_final) return hipSuccess;
        const size_t n = (size_t)a.B * a.H * a.dk * a.dv;
        hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                           dim3(256), 0, (hipStream_t)a.stream, a.s0, a.s_final, n);
        return hipGetLastError();
    }
    return a.bf16 ? launch_chunk_e<kda::bf16>(a) : launch_chunk_e<float>(a);
}

}  // namespace kda
