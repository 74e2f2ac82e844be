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
// The outer factors have exponents bounded by 8 |g_min| (at most 2^93 in
// log2 terms for g_min >= -8, the chunkwise limit).  The middle factor is
// <= 1 but spans 16 or more rows, so alone it can underflow while the key
// factor it multiplies is 2^93: it is applied as its square root twice,
// (k e^{G_m(I) - G_i} s) s with s = e^{(G_m(R) - G_m(I)) / 2}, so that s stays
// normal whenever the product is above 2^-126, and what underflow drops
// stays below 2^-45 after the row factor (at most 2^81).
#include "chunk_layout.hpp"
#include "kda_internal.hpp"

namespace kda {

// ---------------------------------------------------------------------------
// Intra-chunk work of one (b, h, chunk): 256 threads.
//
// Decay exponents are kept in log2 units (G2 = G * log2 e) so that every
// factor is one v_exp_f32.  In phases 1-2 a thread owns two adjacent key
// channels over RP consecutive rows, so global and LDS accesses are packed
// pairs and the row scan runs in registers.
// ---------------------------------------------------------------------------
template <class E, int DK, int DV>
struct Intra {
    typedef typename Compute<E>::type CT;
    static constexpr int CP = DK / 2;        // column pairs
    static constexpr int NPART = 256 / CP;   // row parts (4 or 8)
    static constexpr int RP = C / NPART;     // rows per thread (16 or 8)
    static constexpr int CPV = DV / 2;
    static constexpr int RPV = C / (256 / CPV);
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
    static constexpr size_t OFF_CAR = OFF_DSC;    // scan carries, dead before dsc is written
    static constexpr size_t OFF_GM = OFF_DSC + (NPART > 6 ? NPART : 6) * DK * 4;
    static constexpr size_t OFF_BET = OFF_GM + 5 * DK * 4;
    static constexpr size_t LDS = OFF_BET + C * 4;
    static_assert(RP % 8 == 0 && RPV % 8 == 0 && 16 % RP == 0, "intra tiling");
};

// Block pairs (R, I), I <= R, of A and M handled by each of the 4 waves.
__constant__ int kPairs[4][3][2] = {{{0, 0}, {1, 0}, {3, 3}},
                                    {{1, 1}, {2, 0}, {3, 2}},
                                    {{2, 1}, {2, 2}, {3, 1}},
                                    {{3, 0}, {-1, -1}, {-1, -1}}};

template <class E> __device__ __forceinline__ float dexp2(float x) { return __builtin_amdgcn_exp2f(x); }
template <> __device__ __forceinline__ float dexp2<float>(float x) { return exp2f(x); }

template <class E, int DK, int DV, bool BWD>
__device__ __forceinline__ void intra_chunk(const E* __restrict__ q, const E* __restrict__ k,
                                            const E* __restrict__ v, const E* __restrict__ z,
                                            const E* __restrict__ beta, float g_min, int valid, size_t row0,
                                            int H, unsigned char* __restrict__ blk, unsigned char* smem,
                                            unsigned char* __restrict__ bblk) {
    typedef Intra<E, DK, DV> L;
    typedef typename L::CT CT;
    typedef Mfma<CT> MF;
    typedef Ws<CT, DK, DV> WL;
    constexpr int LDK = L::LDK, LC = L::LC, LA = L::LA, LT = L::LT, RP = L::RP, RPV = L::RPV;
    constexpr float LOG2E = 1.4426950408889634f;

    CT* KL = reinterpret_cast<CT*>(smem);             // [C][LDK] k * e^{G_r - G_m(R)}
    CT* QL = KL + C * LDK;                              // [C][LDK] q * e^{G_r - G_m(R)}
    CT* KR = QL + C * LDK;                              // [C][LDK] k * e^{G_m(R) - G_r}
    float* As = reinterpret_cast<float*>(smem);         // [C][LA]   (after phase 3)
    float* Ts = As + C * LA;                            // [C][LT]
    float* Xs = Ts + C * LT;                            // [3][16][16]
    CT* RT = reinterpret_cast<CT*>(smem + L::OFF_RT);   // [DK][LC] R_K^T = (beta k e^G)^T
    CT* RV = reinterpret_cast<CT*>(smem + L::OFF_RV);   // [DV][LC] R_V^T = (beta v)^T (after phase 3)
    float* dsc = reinterpret_cast<float*>(smem + L::OFF_DSC);   // [6][DK] e^{(G_m(R) - G_m(I)) / 2}
    float* gm = reinterpret_cast<float*>(smem + L::OFF_GM);     // [5][DK] G2_m(R), G2_C
    float* car = reinterpret_cast<float*>(smem + L::OFF_CAR);   // [NPART][DK]
    float* bet = reinterpret_cast<float*>(smem + L::OFF_BET);   // [C]

    CT* gW = reinterpret_cast<CT*>(blk) + WL::W;
    CT* gUT = reinterpret_cast<CT*>(blk) + WL::UT;
    CT* gM = reinterpret_cast<CT*>(blk) + WL::M;
    CT* gQG = reinterpret_cast<CT*>(blk) + WL::QG;
    CT* gKGT = reinterpret_cast<CT*>(blk) + WL::KGT;
    float* gEGC = reinterpret_cast<float*>(reinterpret_cast<CT*>(blk) + WL::END);
    typedef WsB<CT, DK, DV> WB;
    CT* gMT = reinterpret_cast<CT*>(bblk) + WB::MT;
    CT* gKC = reinterpret_cast<CT*>(bblk) + WB::KC;
    CT* gQGT = reinterpret_cast<CT*>(bblk) + WB::QGT;
    CT* gWT = reinterpret_cast<CT*>(bblk) + WB::WT;
    CT* gTT = reinterpret_cast<CT*>(bblk) + WB::TT;
    CT* gAB = reinterpret_cast<CT*>(bblk) + WB::AB;
    constexpr bool BT = BWD && sizeof(CT) == 2;   // T^T and Ab for the bf16 per-chunk gradients

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int last = valid - 1;
    // chunk-base pointers (uniform) and 32-bit per-row offsets
    const E* zb = z + row0 * DK;
    const E* kb = k + row0 * DK;
    const E* qb = q + row0 * DK;
    const E* vb = v + row0 * DV;
    const int rsk = H * DK, rsv = H * DV;

    // ---- phase 1: loads, gate, chunk-local scan of the log2 decay
    if (tid < C) bet[tid] = tid < valid ? to_f32(beta[row0 + (size_t)tid * H]) : 0.f;
    const int c0 = 2 * (tid % L::CP), part = tid / L::CP, r0 = part * RP;
    const int cv0 = 2 * (tid % L::CPV), rv0 = (tid / L::CPV) * RPV;
    typename Pair<E>::type zr[RP], kr[RP], qr[RP], vr[RPV];
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const int off = min(r0 + i, last) * rsk + c0;      // clamped: always in bounds
        zr[i] = load2<E>(zb + off);
        kr[i] = load2<E>(kb + off);
        qr[i] = load2<E>(qb + off);
    }
#pragma unroll
    for (int i = 0; i < RPV; ++i) vr[i] = load2<E>(vb + min(rv0 + i, last) * rsv + cv0);

    const float kg2 = g_min * LOG2E;
    float G[RP][2], kv[RP][2], qv[RP][2];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const bool ok = r0 + i < valid;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float g2 = kg2 * __builtin_amdgcn_rcpf(1.0f + dexp2<E>(-LOG2E * to_f32(zr[i][j])));
            G[i][j] = ok ? g2 : 0.f;
            kv[i][j] = ok ? to_f32(kr[i][j]) : 0.f;
            qv[i][j] = ok ? to_f32(qr[i][j]) : 0.f;
        }
        s0 += G[i][0];
        s1 += G[i][1];
        G[i][0] = s0;
        G[i][1] = s1;
    }
    car[part * DK + c0] = s0;
    car[part * DK + c0 + 1] = s1;
    __syncthreads();
    float cr[2] = {0.f, 0.f}, gC[2] = {0.f, 0.f};
#pragma unroll
    for (int p = 0; p < L::NPART; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float t = car[p * DK + c0 + j];
            if (p < part) cr[j] += t;
            gC[j] += t;     // same summation order as the carry plus the last part's sum
        }
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        G[i][0] += cr[0];
        G[i][1] += cr[1];
        if (((r0 + i) & 15) == 7) {
            gm[((r0 + i) >> 4) * DK + c0] = G[i][0];
            gm[((r0 + i) >> 4) * DK + c0 + 1] = G[i][1];
        }
    }
    if (part == 0) {
        gm[4 * DK + c0] = gC[0];
        gm[4 * DK + c0 + 1] = gC[1];
        gEGC[c0] = dexp2<E>(gC[0]);
        gEGC[c0 + 1] = dexp2<E>(gC[1]);
    }
    __syncthreads();

    // ---- phase 2: decay-scaled operands (the thread's rows lie in one block R)
    {
        const int R = r0 >> 4;
        float gmR[2], eGm[2], eCGm[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            gmR[j] = gm[R * DK + c0 + j];
            eGm[j] = dexp2<E>(gmR[j]);
            eCGm[j] = dexp2<E>(gC[j] - gmR[j]);
        }
        float rk[2][RP], kg[2][RP], qg[BWD ? 2 : 1][BWD ? RP : 1];
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
            float kl[2], ql[2], kR[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float el = G[i][j] - gmR[j];
                const float left = dexp2<E>(el), right = dexp2<E>(-el);
                kl[j] = kv[i][j] * left;
                ql[j] = qv[i][j] * left;
                kR[j] = kv[i][j] * right;
                rk[j][i] = bet[r] * kl[j] * eGm[j];
                kg[j][i] = kR[j] * eCGm[j];
                if constexpr (BWD) qg[j][i] = ql[j] * eGm[j];
            }
            store2<CT>(KL + r * LDK + c0, kl[0], kl[1]);
            store2<CT>(QL + r * LDK + c0, ql[0], ql[1]);
            store2<CT>(KR + r * LDK + c0, kR[0], kR[1]);
            if constexpr (!BWD) store2<CT>(gQG + r * DK + c0, ql[0] * eGm[0], ql[1] * eGm[1]);
            if constexpr (BWD) store2<CT>(gKC + r * DK + c0, kg[0][i], kg[1][i]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < RP; i += 8) {
                store8<CT>(RT + (c0 + j) * LC + r0 + i, &rk[j][i]);
                store8<CT>(gKGT + (c0 + j) * C + r0 + i, &kg[j][i]);
                if constexpr (BWD) store8<CT>(gQGT + (c0 + j) * C + r0 + i, &qg[j][i]);
            }
    }
    for (int idx = tid; idx < 6 * DK; idx += 256) {
        const int p = idx / DK, cc = idx % DK;
        const int R = p < 1 ? 1 : (p < 3 ? 2 : 3);
        const int I = p - R * (R - 1) / 2;
        dsc[idx] = dexp2<E>(0.5f * (gm[R * DK + cc] - gm[I * DK + cc]));   // applied twice
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
#pragma unroll
        for (int kk = 0; kk < DK; kk += MF::KSTEP) {
            typename MF::frag ak = load_frag<CT>(KR, LDK, I * SUB, kk);
            if (I < R) {
                float t[MF::KPL];
                MF::to_floats(ak, t);
                const int cc = kk + (l >> 4) * MF::KPL;
#pragma unroll
                for (int jj = 0; jj < MF::KPL; ++jj) t[jj] = (t[jj] * dv[cc + jj]) * dv[cc + jj];
                ak = MF::from_floats(t);
            }
            accA = MF::mma(ak, load_frag<CT>(KL, LDK, R * SUB, kk), accA);
            accM = MF::mma(ak, load_frag<CT>(QL, LDK, R * SUB, kk), accM);
        }
        const int r = R * SUB + (l & 15);
        const int i0 = I * SUB + 4 * (l >> 4);
        f32x4 mv, abv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            abv[e] = (i0 + e < r) ? accA[e] : 0.f;
            av[j][e] = bet[r] * abv[e];
            mv[e] = (i0 + e <= r) ? accM[e] : 0.f;
        }
        if constexpr (BT) store4<CT>(gAB + r * C + i0, abv);
        if constexpr (!BWD) store4<CT>(gM + r * C + i0, mv);
        if constexpr (BWD) {
#pragma unroll
            for (int e = 0; e < 4; ++e) gMT[(i0 + e) * C + r] = from_f32<CT>(mv[e]);
        }
    }
    if (w == 3) {
        // strictly upper blocks of M are zero
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            const int R = p < 3 ? 0 : (p < 5 ? 1 : 2);
            const int I = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
            if constexpr (!BWD) store4<CT>(gM + (R * SUB + (l & 15)) * C + I * SUB + 4 * (l >> 4), zero4());
            if constexpr (BWD) store4<CT>(gMT + (I * SUB + (l & 15)) * C + R * SUB + 4 * (l >> 4), zero4());
            if constexpr (BT) store4<CT>(gAB + (R * SUB + (l & 15)) * C + I * SUB + 4 * (l >> 4), zero4());
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
    {
        float t0[RPV], t1[RPV];
#pragma unroll
        for (int i = 0; i < RPV; ++i) {
            const float bb = bet[rv0 + i];      // 0 past the end of the sequence
            t0[i] = bb * to_f32(vr[i][0]);
            t1[i] = bb * to_f32(vr[i][1]);
        }
#pragma unroll
        for (int i = 0; i < RPV; i += 8) {
            store8<CT>(RV + cv0 * LC + rv0 + i, &t0[i]);
            store8<CT>(RV + (cv0 + 1) * LC + rv0 + i, &t1[i]);
        }
    }
    __syncthreads();

    // ---- phase 4: T = (I + A)^{-1}, blocked forward substitution
    // 4a: the four unit-lower diagonal blocks I + A_bb, inverted by wave 0,
    //     lane = (block l/16, column l%16), by substitution down the column.
    if (w == 0) {
        const int base = (l >> 4) * SUB, col = l & 15;
        float x[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
            float acc = (r == col) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= As[(base + r) * LA + base + i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < SUB; ++r) Ts[(base + r) * LT + base + col] = x[r];
    } else {
        // waves 1..3 clear the strictly upper blocks (row block R, column block > R)
        for (int i = tid - 64; i < 6 * SUB * SUB; i += 192) {
            const int p = i / (SUB * SUB), e = i % (SUB * SUB);
            const int R = p < 3 ? 0 : (p < 5 ? 1 : 2);
            const int I = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
            Ts[(R * SUB + e / SUB) * LT + I * SUB + e % SUB] = 0.f;
        }
    }
    __syncthreads();
    // 4b: off-diagonal blocks on fp32 MFMA, one block row R at a time; wave I
    //     computes T_RI = -T_RR * sum_{J=I}^{R-1} A_RJ T_JI.
    for (int R = 1; R < 4; ++R) {
        if (w < R) {
            const int I = w;
            f32x4 x = zero4();
            for (int J = I; J < R; ++J)
#pragma unroll
                for (int kk = 0; kk < SUB; kk += 4) {
                    const float a = As[(R * SUB + (l & 15)) * LA + J * SUB + kk + (l >> 4)];
                    const float b = Ts[(J * SUB + kk + (l >> 4)) * LT + I * SUB + (l & 15)];
                    x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, x, 0, 0, 0);
                }
            float* xs = Xs + I * SUB * SUB;
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[(4 * (l >> 4) + e) * SUB + (l & 15)] = x[e];
            f32x4 y = zero4();
#pragma unroll
            for (int kk = 0; kk < SUB; kk += 4) {
                const float a = Ts[(R * SUB + (l & 15)) * LT + R * SUB + kk + (l >> 4)];
                const float b = xs[(kk + (l >> 4)) * SUB + (l & 15)];
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, y, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Ts[(R * SUB + 4 * (l >> 4) + e) * LT + I * SUB + (l & 15)] = -y[e];
        }
        __syncthreads();
    }

    if constexpr (BT) {   // T^T, token index contiguous
        for (int idx = tid; idx < C * (C / 8); idx += 256) {
            const int r = idx % C, a8 = (idx / C) * 8;
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = Ts[(a8 + j) * LT + r];
            store8<CT>(gTT + r * C + a8, t);
        }
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
            if constexpr (BWD) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    gWT[(cb * 16 + 4 * (l >> 4) + e) * C + w * SUB + (l & 15)] = from_f32<CT>(acc[e]);
            }
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

// bws: with BWD, the base of the backward chain's operand blocks (WsB)
template <class E, int DK, int DV, bool BWD = false>
__global__ __launch_bounds__(256) void chunk_intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const E* __restrict__ beta, float g_min, int T, int H, int NC,
    unsigned char* __restrict__ ws, unsigned char* __restrict__ bws = nullptr) {
    typedef typename Compute<E>::type CT;
    extern __shared__ __align__(16) unsigned char smem[];
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t0 = n * C;
    const size_t row0 = ((size_t)b * T + t0) * H + h;
    const size_t cid = ((size_t)b * H + h) * NC + n;
    unsigned char* blk = ws + cid * Ws<CT, DK, DV>::BYTES;
    unsigned char* bblk = BWD ? bws + cid * WsB<CT, DK, DV>::BYTES : nullptr;
    intra_chunk<E, DK, DV, BWD>(q, k, v, z, beta, g_min, min(C, T - t0), row0, H, blk, smem, bblk);
}

// ---------------------------------------------------------------------------
// Chunk-to-chunk recurrence over a range of chunks of one chain (b, h) and
// one tile of TV state columns: 256 threads.
//
//   CM_EXPAND    X starts from the given state; V_new = U - W X; outputs
//                O = (Q e^G) X + M V_new are written; X is the state S.
//   CM_COMPOSE_R X starts from 0 with the same inputs and no outputs: the
//                range's input term R, S_end = P S_start + R.
//   CM_COMPOSE_P X (d_k x d_k) starts from I with no inputs (V_new = -W X):
//                the range's transition P = prod_n (Diag(e^{G_C}) - K~^T W).
// The fp32 X tile lives in MFMA accumulators; each wave loads its operands
// for the next chunk straight from the workspace into registers while the
// current chunk is computed; only X^T and V_new^T go through LDS.
// ---------------------------------------------------------------------------
//   CM_STATES    as CM_EXPAND without outputs, storing instead each chunk's
//                entering state X (fp32) and V_new (compute type): the
//                forward quantities the backward needs (kda_chunk_bwd).
enum { CM_EXPAND = 0, CM_COMPOSE_R = 1, CM_COMPOSE_P = 2, CM_STATES = 3 };

template <class E, int DK, int DV, int NCOL, int TV, int MODE>
struct Chain {
    typedef typename Compute<E>::type CT;
    typedef Mfma<CT> MF;
    static constexpr bool OUT = MODE == CM_EXPAND;
    static constexpr bool HASU = MODE != CM_COMPOSE_P;
    static constexpr int KS = MF::KSTEP;
    static constexpr int NKD = DK / KS;     // k-steps over d_k
    static constexpr int NKC = C / KS;      // k-steps over the chunk's tokens
    static constexpr int RB = DK / 64;      // 16-row state blocks per wave
    static constexpr int NT = TV / 16;      // 16-column tiles
    static constexpr int LDK = DK + 8, LC = C + 8;
    static constexpr size_t SB_BYTES = (size_t)TV * LDK * sizeof(CT);
    static constexpr size_t LDS = 2 * SB_BYTES + (size_t)TV * LC * sizeof(CT);
    static_assert(NCOL % TV == 0 && TV % 16 == 0, "chain tiling");

    // One chunk's operands as held by one wave (rows 16w.. of W, Q*e^G, M;
    // state rows w*DK/4.. of (K*e^{G_C-G})^T; V_new init; e^{G_C}).
    struct Regs {
        typename MF::frag w[NKD], qg[OUT ? NKD : 1], m[OUT ? NKC : 1], kg[RB][NKC];
        typename Raw4<CT>::type u[HASU ? NT : 1];
        f32x4 eg[RB];
    };

    static __device__ __forceinline__ void load(Regs& r, const unsigned char* blk, int w, int l, int col0) {
        typedef Ws<CT, DK, DV> WL;
        const CT* base = reinterpret_cast<const CT*>(blk);
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) {
            r.w[kk] = load_frag<CT>(base + WL::W, DK, w * 16, kk * KS);
            if constexpr (OUT) r.qg[kk] = load_frag<CT>(base + WL::QG, DK, w * 16, kk * KS);
        }
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) {
            if constexpr (OUT) r.m[kk] = load_frag<CT>(base + WL::M, C, w * 16, kk * KS);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                r.kg[rb][kk] = load_frag<CT>(base + WL::KGT, C, w * (DK / 4) + rb * 16, kk * KS);
        }
        if constexpr (HASU) {
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                r.u[ct] = load_raw4<CT>(base + WL::UT + (size_t)(col0 + ct * 16 + (l & 15)) * C + w * 16 + 4 * (l >> 4));
        }
        const float* eg = reinterpret_cast<const float*>(base + WL::END);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            r.eg[rb] = *reinterpret_cast<const f32x4*>(eg + w * (DK / 4) + rb * 16 + 4 * (l >> 4));
    }
};

// One chunk of the recurrence for one wave: consumes the operands in `cur`
// (chunk n) and starts the loads of chunk nfill into `fill`.  The prefetch
// is unconditional (the caller clamps nfill): under a branch the wait-count
// insertion would assume the no-load path and stall on it.
template <class E, int DK, int DV, int NCOL, int TV, int MODE>
__device__ __forceinline__ void chain_step(typename Chain<E, DK, DV, NCOL, TV, MODE>::Regs& cur,
                                           typename Chain<E, DK, DV, NCOL, TV, MODE>::Regs& fill, int n,
                                           int nfill, int T, int H, int b, int h, int col0,
                                           const unsigned char* chain, E* __restrict__ o,
                                           f32x4 (&accS)[DK / 64][TV / 16], typename Compute<E>::type* Sb0,
                                           typename Compute<E>::type* Sb1, typename Compute<E>::type* Vn,
                                           typename Compute<E>::type* __restrict__ st_out,
                                           typename Compute<E>::type* __restrict__ vn_out) {
    typedef Chain<E, DK, DV, NCOL, TV, MODE> L;
    typedef typename L::CT CT;
    typedef typename L::MF MF;
    typedef Ws<CT, DK, DV> WL;
    constexpr int LDK = L::LDK, LC = L::LC, RB = L::RB, NT = L::NT, KS = L::KS;
    const int l = lane_id(), w = wave_id();
    CT* sb = (n & 1) ? Sb1 : Sb0;
    CT* sbn = (n & 1) ? Sb0 : Sb1;
    L::load(fill, chain + (size_t)nfill * WL::BYTES, w, l, col0);
    if constexpr (MODE == CM_STATES) {
        // the state entering chunk n, rows w*DK/4 + rb*16 + 4(l/16) + e
        CT* so = st_out + (size_t)n * DK * DV;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    so[(size_t)(w * (DK / 4) + rb * 16 + 4 * (l >> 4) + e) * DV + col0 + ct * 16 + (l & 15)] =
                        from_f32<CT>(accS[rb][ct][e]);
    }

    // V_new = U - W X (rows 16w.. x TV) and O^T = X^T (Q e^G)^T (TV x rows 16w..)
    f32x4 accP[NT], accO[L::OUT ? NT : 1];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) accP[ct] = zero4();
    if constexpr (L::OUT) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) accO[ct] = zero4();
    }
#pragma unroll
    for (int kk = 0; kk < L::NKD; ++kk)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const typename MF::frag fs = load_frag<CT>(sb, LDK, ct * 16, kk * KS);
            accP[ct] = MF::mma(cur.w[kk], fs, accP[ct]);
            if constexpr (L::OUT) accO[ct] = MF::mma(fs, cur.qg[kk], accO[ct]);
        }
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        f32x4 vn = -accP[ct];
        if constexpr (L::HASU) vn += widen4(cur.u[ct]);
        store4<CT>(Vn + (ct * 16 + (l & 15)) * LC + w * 16 + 4 * (l >> 4), vn);
        if constexpr (MODE == CM_STATES) {
            // V_new row-major, (C, DV) per chunk
            CT* vo = vn_out + (size_t)n * C * DV + (size_t)(w * 16 + 4 * (l >> 4)) * DV + col0 + ct * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) vo[(size_t)e * DV] = from_f32<CT>(vn[e]);
        }
    }
    __syncthreads();

    // O^T += V_new^T M^T ;  X <- Diag(e^{G_C}) X + (K e^{G_C-G})^T V_new
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) accS[rb][ct] *= cur.eg[rb];
#pragma unroll
    for (int kk = 0; kk < L::NKC; ++kk)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const typename MF::frag fv = load_frag<CT>(Vn, LC, ct * 16, kk * KS);
            if constexpr (L::OUT) accO[ct] = MF::mma(fv, cur.m[kk], accO[ct]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) accS[rb][ct] = MF::mma(cur.kg[rb][kk], fv, accS[rb][ct]);
        }
    if constexpr (L::OUT) {
        const int t = n * C + w * 16 + (l & 15);
        if (t < T) {
            E* orow = o + (((size_t)b * T + t) * H + h) * DV + col0;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) store4<E>(orow + ct * 16 + 4 * (l >> 4), accO[ct]);
        }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
            store4<CT>(sbn + (ct * 16 + (l & 15)) * LDK + w * (DK / 4) + rb * 16 + 4 * (l >> 4), accS[rb][ct]);
    __syncthreads();
}

// Grid: 1-D over (tile, segment, chain), tile index major.  Workgroups are
// dealt round-robin to the 8 XCDs, so when B*H*nseg is a multiple of 8 all
// column tiles of one (segment, chain) run on one XCD and share its
// workspace through the same L2.  Segment s covers chunks [sL, min(sL+L, NC)).
//   xin : CM_EXPAND entry states [nseg][B*H][DK][NCOL] (NULL = zeros)
//   xout: CM_EXPAND final state [B*H][DK][NCOL] when nseg == 1 (NULL = skip);
//         CM_COMPOSE_* the range results [nseg][B*H][DK][NCOL]
//   st_out, vn_out: CM_STATES per-chunk entering states [B*H][NC][DK][DV] and
//         V_new [B*H][NC][C][DV] (single level only)
template <class E, int DK, int DV, int NCOL, int TV, int MODE>
__global__ __launch_bounds__(256) void chain_kernel(E* __restrict__ o, const float* __restrict__ xin,
                                                    float* __restrict__ xout, int T, int H, int NC, int L,
                                                    int nchain, const unsigned char* __restrict__ ws,
                                                    typename Compute<E>::type* __restrict__ st_out = nullptr,
                                                    typename Compute<E>::type* __restrict__ vn_out = nullptr) {
    typedef Chain<E, DK, DV, NCOL, TV, MODE> LC_;
    typedef typename LC_::CT CT;
    typedef Ws<CT, DK, DV> WL;
    constexpr int LDK = LC_::LDK, RB = LC_::RB, NT = LC_::NT;

    extern __shared__ __align__(16) unsigned char smem[];
    CT* Sb0 = reinterpret_cast<CT*>(smem);                            // [TV][LDK] X^T, ping
    CT* Sb1 = reinterpret_cast<CT*>(smem + LC_::SB_BYTES);            // pong
    CT* Vn = reinterpret_cast<CT*>(smem + 2 * LC_::SB_BYTES);         // [TV][LC] V_new^T

    const int per_tile = gridDim.x / (NCOL / TV);
    const int tile = blockIdx.x / per_tile;
    const int rem = blockIdx.x % per_tile;
    const int seg = rem / nchain;
    const size_t bh = rem % nchain;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int l = lane_id(), w = wave_id();
    const int col0 = tile * TV;
    const int n0 = seg * L, n1 = min(NC, n0 + L);
    const unsigned char* chain = ws + bh * NC * WL::BYTES;
    const size_t xrow = ((size_t)seg * nchain + bh) * DK;    // row 0 of this (segment, chain) block

    // X rows of this lane: w*DK/4 + rb*16 + 4*(l/16) + e ; column col0 + ct*16 + l%16
    f32x4 accS[RB][NT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int row = w * (DK / 4) + rb * 16 + 4 * (l >> 4);
            const int col = col0 + ct * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = 0.f;
                if constexpr (MODE == CM_EXPAND || MODE == CM_STATES)
                    x = xin ? xin[(xrow + row + e) * NCOL + col] : 0.f;
                if constexpr (MODE == CM_COMPOSE_P) x = (row + e == col) ? 1.f : 0.f;
                accS[rb][ct][e] = x;
            }
            store4<CT>(Sb0 + (ct * 16 + (l & 15)) * LDK + row, accS[rb][ct]);
        }

    // two operand sets: chunk n is consumed while chunk n+1 loads
    CT* st = MODE == CM_STATES ? st_out + bh * NC * DK * DV : nullptr;
    CT* vo = MODE == CM_STATES ? vn_out + bh * NC * C * DV : nullptr;
    typename LC_::Regs r0, r1;
    LC_::load(r0, chain + (size_t)n0 * WL::BYTES, w, l, col0);
    __syncthreads();
    int n = n0;
    for (; n + 2 <= n1; n += 2) {
        chain_step<E, DK, DV, NCOL, TV, MODE>(r0, r1, n, n + 1, T, H, b, h, col0, chain, o, accS, Sb0, Sb1, Vn, st,
                                              vo);
        chain_step<E, DK, DV, NCOL, TV, MODE>(r1, r0, n + 1, min(n + 2, n1 - 1), T, H, b, h, col0, chain, o, accS,
                                              Sb0, Sb1, Vn, st, vo);
    }
    if (n < n1)
        chain_step<E, DK, DV, NCOL, TV, MODE>(r0, r1, n, n, T, H, b, h, col0, chain, o, accS, Sb0, Sb1, Vn, st, vo);

    if (xout) {
        const size_t orow = MODE == CM_EXPAND ? bh * DK : xrow;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const int row = w * (DK / 4) + rb * 16 + 4 * (l >> 4);
                const int col = col0 + ct * 16 + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) xout[(orow + row + e) * NCOL + col] = accS[rb][ct][e];
            }
    }
    (void)LDK;
}

// ---------------------------------------------------------------------------
// Scan over segments for one chain and one tile of TV value columns:
//   Sent[j] = S_j,  S_{j+1} = P_j S_j + R_j,  s_final = S_nseg,
// in fp32 on v_mfma_f32_16x16x4_f32.  The contraction index is visited in
// blocks of 16 as k = 16 kb + 4 g + t (g = lane group, t = sub-step), so each
// lane reads four consecutive entries of a P row (one 16-byte load) and of
// an S^T row in LDS.
// ---------------------------------------------------------------------------
template <int DK, int TV>
struct ScanRegs {
    struct T {
        f32x4 pa[DK / 64][DK / 16];
        float rr[DK / 64][TV / 16][4];
    };
};

template <int DK, int DV, int TV>
__device__ __forceinline__ void scan_fetch(typename ScanRegs<DK, TV>::T& r, const float* __restrict__ P,
                                           const float* __restrict__ R, int j, int nchain, size_t bh, int col0,
                                           int w, int l) {
    constexpr int RB = DK / 64, NT = TV / 16;
    const size_t blk = ((size_t)j * nchain + bh) * DK;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
            r.pa[rb][kb] = *reinterpret_cast<const f32x4*>(P + (blk + w * (DK / 4) + rb * 16 + (l & 15)) * DK +
                                                            kb * 16 + 4 * (l >> 4));
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r.rr[rb][ct][e] = R[(blk + w * (DK / 4) + rb * 16 + 4 * (l >> 4) + e) * DV + col0 + ct * 16 + (l & 15)];
    }
}

// One segment of the scan: Sent[j] = S; S <- P_j S + R_j (operands in `cur`),
// while segment jn's operands load into `nxt`.
template <int DK, int DV, int TV>
__device__ __forceinline__ void scan_step(f32x4 (&acc)[DK / 64][TV / 16], typename ScanRegs<DK, TV>::T& cur,
                                          typename ScanRegs<DK, TV>::T& nxt, const float* __restrict__ P,
                                          const float* __restrict__ R, float* __restrict__ Sent, float* St, int j,
                                          int jn, int nchain, size_t bh, int col0, int w, int l) {
    constexpr int RB = DK / 64, NT = TV / 16, LS = DK + 4;
    scan_fetch<DK, DV, TV>(nxt, P, R, jn, nchain, bh, col0, w, l);
    const size_t blk = ((size_t)j * nchain + bh) * DK;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int row = w * (DK / 4) + rb * 16 + 4 * (l >> 4);
            const int col = ct * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) Sent[(blk + row + e) * DV + col0 + col] = acc[rb][ct][e];
            *reinterpret_cast<f32x4*>(St + col * LS + row) = acc[rb][ct];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rb][ct][e] = cur.rr[rb][ct][e];   // accumulate onto R_j
        }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < DK / 16; ++kb) {
        f32x4 sv[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
            sv[ct] = *reinterpret_cast<const f32x4*>(St + (ct * 16 + (l & 15)) * LS + kb * 16 + 4 * (l >> 4));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
                    acc[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.pa[rb][kb][t], sv[ct][t], acc[rb][ct], 0, 0, 0);
    }
    __syncthreads();
}

template <int DK, int DV, int TV>
__global__ __launch_bounds__(256) void seg_scan_kernel(const float* __restrict__ P, const float* __restrict__ R,
                                                       const float* __restrict__ s0, float* __restrict__ Sent,
                                                       float* __restrict__ s_final, int nseg, int nchain) {
    constexpr int RB = DK / 64, NT = TV / 16, LS = DK + 4;
    __shared__ __align__(16) float St[TV * LS];     // S^T tile
    const int tile = blockIdx.x / nchain;
    const size_t bh = blockIdx.x % nchain;
    const int l = lane_id(), w = wave_id();
    const int col0 = tile * TV;

    f32x4 acc[RB][NT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = w * (DK / 4) + rb * 16 + 4 * (l >> 4) + e;
                acc[rb][ct][e] = s0 ? s0[(bh * DK + row) * DV + col0 + ct * 16 + (l & 15)] : 0.f;
            }
    // P_j rows of this wave and the R_j tile, prefetched one segment ahead in
    // two register sets (a / b, explicitly unrolled: no dynamic indexing)
    typename ScanRegs<DK, TV>::T ra, rb_;
    scan_fetch<DK, DV, TV>(ra, P, R, 0, nchain, bh, col0, w, l);
    int j = 0;
    for (; j + 2 <= nseg; j += 2) {
        scan_step<DK, DV, TV>(acc, ra, rb_, P, R, Sent, St, j, j + 1, nchain, bh, col0, w, l);
        scan_step<DK, DV, TV>(acc, rb_, ra, P, R, Sent, St, j + 1, min(j + 2, nseg - 1), nchain, bh, col0, w, l);
    }
    if (j < nseg) scan_step<DK, DV, TV>(acc, ra, rb_, P, R, Sent, St, j, j, nchain, bh, col0, w, l);
    if (s_final) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = w * (DK / 4) + rb * 16 + 4 * (l >> 4) + e;
                    s_final[(bh * DK + row) * DV + col0 + ct * 16 + (l & 15)] = acc[rb][ct][e];
                }
    }
}

// State pass-through for T == 0: s_final = s0 (or zeros).
__global__ void state_copy_kernel(const float* __restrict__ s0, float* __restrict__ s_final, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        s_final[i] = s0 ? s0[i] : 0.f;
}

// ---------------------------------------------------------------------------
// Sequences of at least 2*SEG_L chunks use two levels (compose / scan /
// expand over segments of SEG_L chunks); shorter ones one chain per tile.
constexpr int SEG_L = 16;

struct Layout {
    size_t chunks, p_off, r_off, e_off, total;
    int nseg;
};

template <class CT, int DK, int DV>
static Layout layout_t(int B, int T, int H) {
    Layout lo{};
    const size_t NC = ((size_t)T + C - 1) / C;
    const size_t nchain = (size_t)B * H;
    lo.chunks = nchain * NC * Ws<CT, DK, DV>::BYTES;
    lo.nseg = NC >= 2 * SEG_L ? (int)((NC + SEG_L - 1) / SEG_L) : 1;
    lo.p_off = lo.r_off = lo.e_off = lo.total = lo.chunks;
    if (lo.nseg > 1) {
        lo.r_off = lo.p_off + (size_t)lo.nseg * nchain * DK * DK * 4;
        lo.e_off = lo.r_off + (size_t)lo.nseg * nchain * DK * DV * 4;
        lo.total = lo.e_off + (size_t)lo.nseg * nchain * DK * DV * 4;
    }
    return lo;
}

template <class K>
static hipError_t set_lds(K kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <class E, int DK, int DV>
static hipError_t launch_chunk_t(const ChunkArgs& a) {
    typedef typename Compute<E>::type CT;
    constexpr bool BF = sizeof(CT) == 2;
    constexpr int TVS = BF ? 32 : 16;          // single level: more chains on the chip
    constexpr int TVV = BF ? DV : 16;          // two level: one read of the operands per chunk
    constexpr int TVK = BF ? DK : 16;
    const int NC = (a.T + C - 1) / C;
    const int nchain = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    typedef Intra<E, DK, DV> LI;
    static_assert(LI::LDS <= 160 * 1024, "intra LDS budget");
    const Layout lo = layout_t<CT, DK, DV>(a.B, a.T, a.H);
    unsigned char* ws = (unsigned char*)a.workspace;
    hipError_t err = set_lds(chunk_intra_kernel<E, DK, DV>, LI::LDS);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((chunk_intra_kernel<E, DK, DV>), dim3(NC, a.H, a.B), dim3(256), LI::LDS, st,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta,
                       a.g_min, a.T, a.H, NC, ws);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    if (lo.nseg == 1) {
        typedef Chain<E, DK, DV, DV, TVS, CM_EXPAND> LX;
        if ((err = set_lds(chain_kernel<E, DK, DV, DV, TVS, CM_EXPAND>, LX::LDS)) != hipSuccess) return err;
        hipLaunchKernelGGL((chain_kernel<E, DK, DV, DV, TVS, CM_EXPAND>), dim3((DV / TVS) * nchain), dim3(256),
                           LX::LDS, st, (E*)a.o, a.s0, a.s_final, a.T, a.H, NC, NC, nchain,
                           (const unsigned char*)ws);
        return hipGetLastError();
    }
    float* Pb = reinterpret_cast<float*>(ws + lo.p_off);
    float* Rb = reinterpret_cast<float*>(ws + lo.r_off);
    float* Eb = reinterpret_cast<float*>(ws + lo.e_off);
    const int nseg = lo.nseg;
    typedef Chain<E, DK, DV, DV, TVV, CM_COMPOSE_R> LR;
    typedef Chain<E, DK, DV, DK, TVK, CM_COMPOSE_P> LP;
    typedef Chain<E, DK, DV, DV, TVV, CM_EXPAND> LE;
    if ((err = set_lds(chain_kernel<E, DK, DV, DV, TVV, CM_COMPOSE_R>, LR::LDS)) != hipSuccess) return err;
    if ((err = set_lds(chain_kernel<E, DK, DV, DK, TVK, CM_COMPOSE_P>, LP::LDS)) != hipSuccess) return err;
    if ((err = set_lds(chain_kernel<E, DK, DV, DV, TVV, CM_EXPAND>, LE::LDS)) != hipSuccess) return err;
    hipLaunchKernelGGL((chain_kernel<E, DK, DV, DK, TVK, CM_COMPOSE_P>), dim3((DK / TVK) * nseg * nchain), dim3(256),
                       LP::LDS, st, (E*)nullptr, (const float*)nullptr, Pb, a.T, a.H, NC, SEG_L, nchain,
                       (const unsigned char*)ws);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((chain_kernel<E, DK, DV, DV, TVV, CM_COMPOSE_R>), dim3((DV / TVV) * nseg * nchain), dim3(256),
                       LR::LDS, st, (E*)nullptr, (const float*)nullptr, Rb, a.T, a.H, NC, SEG_L, nchain,
                       (const unsigned char*)ws);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV, 32>), dim3((DV / 32) * nchain), dim3(256), 0, st, Pb, Rb, a.s0, Eb,
                       a.s_final, nseg, nchain);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((chain_kernel<E, DK, DV, DV, TVV, CM_EXPAND>), dim3((DV / TVV) * nseg * nchain), dim3(256),
                       LE::LDS, st, (E*)a.o, (const float*)Eb, (float*)nullptr, a.T, a.H, NC, SEG_L, nchain,
                       (const unsigned char*)ws);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_chunk_e(const ChunkArgs& a) {
    if (a.dk == 128 && a.dv == 128) return launch_chunk_t<E, 128, 128>(a);
    if (a.dk == 128 && a.dv == 64) return launch_chunk_t<E, 128, 64>(a);
    if (a.dk == 64 && a.dv == 128) return launch_chunk_t<E, 64, 128>(a);
    return launch_chunk_t<E, 64, 64>(a);
}

template <class CT>
static size_t ws_bytes_t(int B, int T, int H, int dk, int dv) {
    if (dk == 128 && dv == 128) return layout_t<CT, 128, 128>(B, T, H).total;
    if (dk == 128 && dv == 64) return layout_t<CT, 128, 64>(B, T, H).total;
    if (dk == 64 && dv == 128) return layout_t<CT, 64, 128>(B, T, H).total;
    return layout_t<CT, 64, 64>(B, T, H).total;
}

size_t chunk_workspace_bytes(int B, int T, int H, int dk, int dv, bool bf16) {
    return bf16 ? seg_workspace_bytes(B, T, H, dk, dv) : ws_bytes_t<float>(B, T, H, dk, dv);
}

template <int DK, int DV>
static hipError_t launch_scan_t(const float* P, const float* R, const float* s0, float* Sent, float* s_final,
                                int nseg, int nchain, hipStream_t st) {
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV, 16>), dim3((DV / 16) * nchain), dim3(256), 0, st, P, R, s0, Sent,
                       s_final, nseg, nchain);
    return hipGetLastError();
}

hipError_t launch_seg_scan(const float* P, const float* R, const float* s0, float* Sent, float* s_final, int nseg,
                           int nchain, int dk, int dv, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (dk == 128 && dv == 128) return launch_scan_t<128, 128>(P, R, s0, Sent, s_final, nseg, nchain, st);
    if (dk == 128 && dv == 64) return launch_scan_t<128, 64>(P, R, s0, Sent, s_final, nseg, nchain, st);
    if (dk == 64 && dv == 128) return launch_scan_t<64, 128>(P, R, s0, Sent, s_final, nseg, nchain, st);
    return launch_scan_t<64, 64>(P, R, s0, Sent, s_final, nseg, nchain, st);
}

// The forward half of kda_chunk_bwd: the per-chunk operands of both
// directions (fws: Ws blocks, bws: WsB blocks), then the chunk recurrence
// from s0 storing each chunk's entering state and V_new.
template <class E, int DK, int DV>
static hipError_t launch_bwd_forward_t(const BwdArgs& a, unsigned char* fws, unsigned char* bws, void* states,
                                       void* vn) {
    typedef typename Compute<E>::type CT;
    // bf16: one workgroup per chain over all value columns, so each chunk's W and
    // (K e^{G_C-G})^T are read once (8.3 against 9.1 ms for 32-column tiles at 8x8192x32)
    constexpr int TVS = sizeof(CT) == 2 ? (DV < 128 ? DV : 128) : 16;
    const int NC = (a.T + C - 1) / C;
    const int nchain = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    typedef Intra<E, DK, DV> LI;
    hipError_t err = set_lds(chunk_intra_kernel<E, DK, DV, true>, LI::LDS);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((chunk_intra_kernel<E, DK, DV, true>), dim3(NC, a.H, a.B), dim3(256), LI::LDS, st,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.T,
                       a.H, NC, fws, bws);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    typedef Chain<E, DK, DV, DV, TVS, CM_STATES> LX;
    if ((err = set_lds(chain_kernel<E, DK, DV, DV, TVS, CM_STATES>, LX::LDS)) != hipSuccess) return err;
    hipLaunchKernelGGL((chain_kernel<E, DK, DV, DV, TVS, CM_STATES>), dim3((DV / TVS) * nchain), dim3(256), LX::LDS,
                       st, (E*)nullptr, a.s0, (float*)nullptr, a.T, a.H, NC, NC, nchain, (const unsigned char*)fws,
                       (CT*)states, (CT*)vn);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_bwd_forward_e(const BwdArgs& a, unsigned char* fws, unsigned char* bws, void* states,
                                       void* vn) {
    if (a.dk_dim == 128 && a.dv_dim == 128) return launch_bwd_forward_t<E, 128, 128>(a, fws, bws, states, vn);
    if (a.dk_dim == 128 && a.dv_dim == 64) return launch_bwd_forward_t<E, 128, 64>(a, fws, bws, states, vn);
    if (a.dk_dim == 64 && a.dv_dim == 128) return launch_bwd_forward_t<E, 64, 128>(a, fws, bws, states, vn);
    return launch_bwd_forward_t<E, 64, 64>(a, fws, bws, states, vn);
}

hipError_t launch_chunk_bwd_forward(const BwdArgs& a, unsigned char* fws, unsigned char* bws, void* states,
                                    void* vn) {
    return a.bf16 ? launch_bwd_forward_e<bf16>(a, fws, bws, states, vn)
                  : launch_bwd_forward_e<float>(a, fws, bws, states, vn);
}

hipError_t launch_chunk(const ChunkArgs& a) {
    if (a.T == 0) {
        if (!a.s_final) return hipSuccess;
        const size_t n = (size_t)a.B * a.H * a.dk * a.dv;
        hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                           dim3(256), 0, (hipStream_t)a.stream, a.s0, a.s_final, n);
        return hipGetLastError();
    }
    if (a.g_min < CHUNK_G_MIN_LIMIT) return launch_seq(a);
    return a.bf16 ? launch_chunk_seg(a) : launch_chunk_e<float>(a);
}

}  // namespace kda
