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
// The unit-lower system I + A is solved without a dense inverse of the full
// system by blocked forward substitution on 16x16 blocks (the triangular
// factor T = (I + A)^{-1} is itself lower triangular), then W = T R_K and
// U = T R_V are two MFMA products.
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
//    The fp32 state tile lives in MFMA accumulators for the whole sequence.
//
// Overflow: e^{G_r - G_i} is never formed as e^{G_r} e^{-G_i} over the whole
// chunk (|G| reaches 64 * |g_min|, far beyond the fp32 range).  A and M are
// evaluated per 16x16 block (R, I) with a reference row m inside row block R:
// e^{G_r - G_i} = e^{G_r - G_m} * e^{G_m - G_i}.  For I < R both factors are
// <= 1; for I = R both exponents are bounded by 8 * |g_min|.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

constexpr int C = 64;     // chunk length
constexpr int SUB = 16;   // block size of the triangular solve and of A / M

template <class E> struct Compute { typedef bf16 type; };
template <> struct Compute<float> { typedef float type; };

// exp for decay factors: the correctly rounded-ish libm exp on the fp32 path,
// the hardware exp2-based one on the bf16 path.
template <class E> __device__ __forceinline__ float dexp(float x) { return __expf(x); }
template <> __device__ __forceinline__ float dexp<float>(float x) { return expf(x); }

// Workspace block of one (b, h, chunk), in elements of the compute type CT
// unless noted; every part starts on a 16-byte boundary.
template <class CT, int DK, int DV>
struct Ws {
    static constexpr size_t W = 0;                    // (C, DK)   row-major
    static constexpr size_t U = W + (size_t)C * DK;   // (C, DV)
    static constexpr size_t M = U + (size_t)C * DV;   // (C, C)
    static constexpr size_t QG = M + (size_t)C * C;   // (C, DK)   q * e^{G}
    static constexpr size_t KGT = QG + (size_t)C * DK;// (DK, C)   (k * e^{G_C - G})^T
    static constexpr size_t END = KGT + (size_t)DK * C;
    static constexpr size_t BYTES = END * sizeof(CT) + DK * sizeof(float);  // + e^{G_C} fp32
};

// Copy a rows x cols tile (cols a multiple of 16 bytes) from global to LDS
// with 16-byte accesses, all threads of the block cooperating.
template <class CT>
__device__ __forceinline__ void copy_tile(CT* dst, int ldd, const CT* src, int lds, int rows, int cols) {
    constexpr int VE = 16 / sizeof(CT);
    const int vpr = cols / VE;
    const int nv = rows * vpr;
    for (int i = threadIdx.x; i < nv; i += blockDim.x) {
        const int r = i / vpr, cv = i % vpr;
        *reinterpret_cast<u32x4*>(dst + (size_t)r * ldd + cv * VE) =
            *reinterpret_cast<const u32x4*>(src + (size_t)r * lds + cv * VE);
    }
}

// ---------------------------------------------------------------------------
// Intra-chunk kernel
// ---------------------------------------------------------------------------
template <class E, int DK, int DV>
struct IntraSmem {
    typedef typename Compute<E>::type CT;
    static constexpr int LG = DK + 1;     // Gs row stride (floats)
    static constexpr int LDK = DK + 8;    // Ks row stride (CT)
    static constexpr int LC = C + 8;      // RT row stride (CT)
    static constexpr int LA = C + 1;      // As row stride (floats)
    static constexpr int LT = C + 4;      // Ts row stride (floats)
    static constexpr size_t G_BYTES = (size_t)C * LG * 4;
    static constexpr size_t K_BYTES = ((size_t)C * LDK * sizeof(CT) + 15) / 16 * 16;
    static constexpr size_t A_BYTES = ((size_t)C * LA * 4 + 15) / 16 * 16;
    static constexpr size_t T_BYTES = (size_t)C * LT * 4;
    static constexpr size_t X_BYTES = (G_BYTES + K_BYTES) > (A_BYTES + T_BYTES + 3 * SUB * SUB * 4)
                                          ? (G_BYTES + K_BYTES) : (A_BYTES + T_BYTES + 3 * SUB * SUB * 4);
    static constexpr size_t RT_OFF = (X_BYTES + 15) / 16 * 16;
    static constexpr size_t RT_BYTES = (size_t)(DK + DV) * LC * sizeof(CT);
    static constexpr size_t BET_OFF = RT_OFF + RT_BYTES;
    static constexpr size_t TOTAL = BET_OFF + C * 4;
};

template <class E, int DK, int DV>
__global__ __launch_bounds__(256) void chunk_intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ z, const E* __restrict__ beta, float g_min, int T, int H, int NC,
    unsigned char* __restrict__ ws) {
    typedef typename Compute<E>::type CT;
    typedef Mfma<CT> MF;
    typedef IntraSmem<E, DK, DV> L;
    typedef Ws<CT, DK, DV> WL;
    constexpr int LG = L::LG, LDK = L::LDK, LC = L::LC, LA = L::LA, LT = L::LT;
    constexpr int NPART = 256 / DK;       // threads per channel in the scan
    constexpr int RP = C / NPART;         // rows per scan part

    extern __shared__ __align__(16) unsigned char smem[];
    float* Gs = reinterpret_cast<float*>(smem);                          // [C][LG]
    CT* Ks = reinterpret_cast<CT*>(smem + L::G_BYTES);                   // [C][LDK]
    float* As = reinterpret_cast<float*>(smem);                          // [C][LA]   (after phase 3)
    float* Ts = reinterpret_cast<float*>(smem + L::A_BYTES);             // [C][LT]
    float* Xs = Ts + C * LT;                                             // [3][16][16]
    CT* RT = reinterpret_cast<CT*>(smem + L::RT_OFF);                    // [DK+DV][LC]
    float* bet = reinterpret_cast<float*>(smem + L::BET_OFF);            // [C]

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int t0 = n * C;
    const int valid = min(C, T - t0);
    const size_t row0 = ((size_t)b * T + t0) * H + h;   // token row (b, t0, h)
    const size_t rstride = H;                            // token-row step per t
    unsigned char* blk = ws + (((size_t)b * H + h) * NC + n) * WL::BYTES;
    CT* gW = reinterpret_cast<CT*>(blk) + WL::W;
    CT* gU = reinterpret_cast<CT*>(blk) + WL::U;
    CT* gM = reinterpret_cast<CT*>(blk) + WL::M;
    CT* gQG = reinterpret_cast<CT*>(blk) + WL::QG;
    CT* gKGT = reinterpret_cast<CT*>(blk) + WL::KGT;
    float* gEGC = reinterpret_cast<float*>(reinterpret_cast<CT*>(blk) + WL::END);

    // ---- phase 1: g = g_min * sigmoid(z), chunk-local inclusive scan -> Gs
    if (tid < C) bet[tid] = tid < valid ? to_f32(beta[row0 + tid * rstride]) : 0.f;
    for (int i = tid; i < C * DK; i += 256) {
        const int r = i / DK, c = i % DK;
        float g = 0.f;
        if (r < valid) g = g_min * sigmoidf_(to_f32(z[(row0 + r * rstride) * DK + c]));
        Gs[r * LG + c] = g;
    }
    __syncthreads();
    {
        const int c = tid % DK, part = tid / DK;
        float s = 0.f;
        for (int i = 0; i < RP; ++i) {
            const int r = part * RP + i;
            s += Gs[r * LG + c];
            Gs[r * LG + c] = s;
        }
    }
    __syncthreads();
    {
        const int c = tid % DK, part = tid / DK;
        float carry = 0.f;
        for (int p = 0; p < part; ++p) carry += Gs[(p * RP + RP - 1) * LG + c];
        __syncthreads();
        if (part > 0)
            for (int i = 0; i < RP; ++i) Gs[(part * RP + i) * LG + c] += carry;
    }
    __syncthreads();

    // ---- phase 2: elementwise decay factors
    for (int i = tid; i < C * DK; i += 256) {
        const int r = i / DK, c = i % DK;
        float kv = 0.f, qv = 0.f;
        if (r < valid) {
            kv = to_f32(k[(row0 + r * rstride) * DK + c]);
            qv = to_f32(q[(row0 + r * rstride) * DK + c]);
        }
        const float eg = dexp<E>(Gs[r * LG + c]);
        Ks[r * LDK + c] = from_f32<CT>(kv);
        gQG[r * DK + c] = from_f32<CT>(qv * eg);
        RT[c * LC + r] = from_f32<CT>(bet[r] * kv * eg);
    }
    for (int i = tid; i < C * DV; i += 256) {
        const int r = i / DV, c = i % DV;
        const float vv = r < valid ? to_f32(v[(row0 + r * rstride) * DV + c]) : 0.f;
        RT[(DK + c) * LC + r] = from_f32<CT>(bet[r] * vv);
    }
    if (tid < DK) gEGC[tid] = dexp<E>(Gs[(C - 1) * LG + tid]);
    __syncthreads();
    for (int i = tid; i < C * DK; i += 256) {
        const int c = i / C, r = i % C;
        const float gc = Gs[(C - 1) * LG + c];
        gKGT[c * C + r] = from_f32<CT>(to_f32(Ks[r * LDK + c]) * dexp<E>(gc - Gs[r * LG + c]));
    }

    // ---- phase 3: A and M, 16x16 blocks (R = this wave's row block, I <= R)
    float aval[4][4];
    {
        const int R = w;
        const int m = R * SUB + SUB / 2 - 1;           // reference row of block R
        const int rr = R * SUB + (l & 15);              // A-operand row of this lane
        for (int I = 0; I < 4; ++I) {
            f32x4 accA = zero4(), accM = zero4();
            if (I <= R) {
                const int ii = I * SUB + (l & 15);      // B-operand row (key index)
                for (int kk = 0; kk < DK; kk += MF::KSTEP) {
                    const int c0 = kk + (l >> 4) * MF::KPL;
                    float ak[MF::KPL], aq[MF::KPL], bk[MF::KPL];
#pragma unroll
                    for (int j = 0; j < MF::KPL; ++j) {
                        const float gm = Gs[m * LG + c0 + j];
                        const float fl = dexp<E>(Gs[rr * LG + c0 + j] - gm);
                        const float fr = dexp<E>(gm - Gs[ii * LG + c0 + j]);
                        const float qv = rr < valid ? to_f32(q[(row0 + rr * rstride) * DK + c0 + j]) : 0.f;
                        ak[j] = to_f32(Ks[rr * LDK + c0 + j]) * fl;
                        aq[j] = qv * fl;
                        bk[j] = to_f32(Ks[ii * LDK + c0 + j]) * fr;
                    }
                    const typename MF::frag fa = MF::from_floats(ak), fq = MF::from_floats(aq),
                                            fb = MF::from_floats(bk);
                    accA = MF::mma(fa, fb, accA);
                    accM = MF::mma(fq, fb, accM);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = R * SUB + acc_row(e);
                const int i = I * SUB + acc_col();
                aval[I][e] = i < r ? bet[r] * accA[e] : 0.f;
                gM[r * C + i] = from_f32<CT>(i <= r ? accM[e] : 0.f);
            }
        }
    }
    __syncthreads();   // Gs / Ks are dead from here on; As and Ts alias them
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) As[(w * SUB + acc_row(e)) * LA + I * SUB + acc_col()] = aval[I][e];
    __syncthreads();

    // ---- phase 4: T = (I + A)^{-1}, blocked forward substitution
    // 4a: diagonal blocks, wave w inverts I + A_ww column by column.
    if (l < SUB) {
        const int base = w * SUB;
        float x[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
            float s = (r == l) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s -= As[(base + r) * LA + base + i] * x[i];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < SUB; ++r) Ts[(base + r) * LT + base + l] = x[r];
    } else {
        // the remaining lanes clear the blocks right of the diagonal block
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
            float s = 0.f;
            for (int J = I; J < R; ++J)
#pragma unroll
                for (int t = 0; t < SUB; ++t)
                    s += As[(R * SUB + rl) * LA + J * SUB + t] * Ts[(J * SUB + t) * LT + I * SUB + il];
            Xs[(I * SUB + rl) * SUB + il] = s;
        }
        __syncthreads();
        for (int I = 0; I < R; ++I) {
            float s = 0.f;
#pragma unroll
            for (int t = 0; t < SUB; ++t)
                s -= Ts[(R * SUB + rl) * LT + R * SUB + t] * Xs[(I * SUB + t) * SUB + il];
            Ts[(R * SUB + rl) * LT + I * SUB + il] = s;
        }
        __syncthreads();
    }

    // ---- phase 5: [W | U] = T [R_K | R_V]; wave w computes row block w
    {
        const int R = w;
        constexpr int NKS = C / MF::KSTEP;
        typename MF::frag ta[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) ta[s] = load_frag_f32<CT>(Ts, LT, R * SUB, s * MF::KSTEP);
        const int kend = (R + 1) * SUB;                 // T_R. is zero beyond column kend
        for (int ct = 0; ct < (DK + DV) / 16; ++ct) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                if (s * MF::KSTEP < kend) acc = MF::mma(ta[s], load_frag<CT>(RT, LC, ct * 16, s * MF::KSTEP), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = R * SUB + acc_row(e);
                const int c = ct * 16 + acc_col();
                if (c < DK) gW[r * DK + c] = from_f32<CT>(acc[e]);
                else gU[r * DV + (c - DK)] = from_f32<CT>(acc[e]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Inter-chunk kernel
// ---------------------------------------------------------------------------
template <class E, int DK, int DV, int TV>
struct InterSmem {
    typedef typename Compute<E>::type CT;
    static constexpr int LDK = DK + 8, LC = C + 8;
    static constexpr size_t W_OFF = 0;
    static constexpr size_t Q_OFF = W_OFF + (size_t)C * LDK * sizeof(CT);
    static constexpr size_t KT_OFF = Q_OFF + (size_t)C * LDK * sizeof(CT);
    static constexpr size_t M_OFF = KT_OFF + (size_t)DK * LC * sizeof(CT);
    static constexpr size_t U_OFF = M_OFF + (size_t)C * LC * sizeof(CT);
    static constexpr size_t EG_OFF = U_OFF + (size_t)C * TV * sizeof(CT);
    static constexpr size_t SB_OFF = EG_OFF + DK * 4;
    static constexpr size_t VN_OFF = SB_OFF + (size_t)TV * LDK * sizeof(CT);
    static constexpr size_t TOTAL = VN_OFF + (size_t)TV * LC * sizeof(CT);
};

template <class E, int DK, int DV, int TV>
__global__ __launch_bounds__(256) void chunk_inter_kernel(
    E* __restrict__ o, const float* __restrict__ s0, float* __restrict__ s_final, int T, int H,
    int NC, const unsigned char* __restrict__ ws) {
    typedef typename Compute<E>::type CT;
    typedef Mfma<CT> MF;
    typedef InterSmem<E, DK, DV, TV> L;
    typedef Ws<CT, DK, DV> WL;
    constexpr int LDK = L::LDK, LC = L::LC;
    constexpr int NT = TV / 16;       // column tiles per workgroup
    constexpr int RB = DK / 64;       // 16-row state blocks per wave

    extern __shared__ __align__(16) unsigned char smem[];
    CT* Wsm = reinterpret_cast<CT*>(smem + L::W_OFF);
    CT* Qsm = reinterpret_cast<CT*>(smem + L::Q_OFF);
    CT* KTs = reinterpret_cast<CT*>(smem + L::KT_OFF);
    CT* Msm = reinterpret_cast<CT*>(smem + L::M_OFF);
    CT* Usm = reinterpret_cast<CT*>(smem + L::U_OFF);
    float* eG = reinterpret_cast<float*>(smem + L::EG_OFF);
    CT* Sb = reinterpret_cast<CT*>(smem + L::SB_OFF);    // [TV][LDK]  S^T in operand precision
    CT* Vn = reinterpret_cast<CT*>(smem + L::VN_OFF);    // [TV][LC]   V_new^T

    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = wave_id();
    const int col0 = tile * TV;
    const size_t bh = (size_t)b * H + h;

    // state tile rows owned by this wave: w*DK/4 + rb*16 + acc_row(e)
    f32x4 accS[RB][NT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = w * (DK / 4) + rb * 16 + acc_row(e);
                const int col = ct * 16 + acc_col();
                const float sv = s0 ? s0[(bh * DK + row) * DV + col0 + col] : 0.f;
                accS[rb][ct][e] = sv;
                Sb[col * LDK + row] = from_f32<CT>(sv);
            }

    for (int n = 0; n < NC; ++n) {
        const CT* blk = reinterpret_cast<const CT*>(ws + (bh * NC + n) * WL::BYTES);
        copy_tile<CT>(Wsm, LDK, blk + WL::W, DK, C, DK);
        copy_tile<CT>(Qsm, LDK, blk + WL::QG, DK, C, DK);
        copy_tile<CT>(KTs, LC, blk + WL::KGT, C, DK, C);
        copy_tile<CT>(Msm, LC, blk + WL::M, C, C, C);
        copy_tile<CT>(Usm, TV, blk + WL::U + col0, DV, C, TV);
        if (threadIdx.x < DK) eG[threadIdx.x] = reinterpret_cast<const float*>(blk + WL::END)[threadIdx.x];
        __syncthreads();

        // V_new = U - W S and Q*e^G S for token rows 16w .. 16w+15
        f32x4 accP[NT], accO[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) { accP[ct] = zero4(); accO[ct] = zero4(); }
        for (int kk = 0; kk < DK; kk += MF::KSTEP) {
            const typename MF::frag fw = load_frag<CT>(Wsm, LDK, w * 16, kk);
            const typename MF::frag fq = load_frag<CT>(Qsm, LDK, w * 16, kk);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const typename MF::frag fs = load_frag<CT>(Sb, LDK, ct * 16, kk);
                accP[ct] = MF::mma(fw, fs, accP[ct]);
                accO[ct] = MF::mma(fq, fs, accO[ct]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = w * 16 + acc_row(e);
                const int c = ct * 16 + acc_col();
                const float vn = to_f32(Usm[r * TV + c]) - accP[ct][e];
                Vn[c * LC + r] = from_f32<CT>(vn);
            }
        __syncthreads();

        // O = Q*e^G S + M V_new
        for (int kk = 0; kk < C; kk += MF::KSTEP) {
            const typename MF::frag fm = load_frag<CT>(Msm, LC, w * 16, kk);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                accO[ct] = MF::mma(fm, load_frag<CT>(Vn, LC, ct * 16, kk), accO[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = w * 16 + acc_row(e);
                const int t = n * C + r;
                if (t < T) o[(((size_t)b * T + t) * H + h) * DV + col0 + ct * 16 + acc_col()] = from_f32<E>(accO[ct][e]);
            }

        // S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T V_new
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = eG[w * (DK / 4) + rb * 16 + acc_row(e)];
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) accS[rb][ct][e] *= f;
            }
        for (int kk = 0; kk < C; kk += MF::KSTEP) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const typename MF::frag fk = load_frag<CT>(KTs, LC, w * (DK / 4) + rb * 16, kk);
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
                    accS[rb][ct] = MF::mma(fk, load_frag<CT>(Vn, LC, ct * 16, kk), accS[rb][ct]);
            }
        }
        __syncthreads();   // all reads of Vn, Sb and the chunk tiles are done
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Sb[(ct * 16 + acc_col()) * LDK + w * (DK / 4) + rb * 16 + acc_row(e)] =
                        from_f32<CT>(accS[rb][ct][e]);
    }

    if (s_final) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = w * (DK / 4) + rb * 16 + acc_row(e);
                    s_final[(bh * DK + row) * DV + col0 + ct * 16 + acc_col()] = accS[rb][ct][e];
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
    typedef IntraSmem<E, DK, DV> LI;
    typedef InterSmem<E, DK, DV, TV> LX;
    static_assert(LI::TOTAL <= 160 * 1024, "intra LDS budget");
    static_assert(LX::TOTAL <= 160 * 1024, "inter LDS budget");
    hipError_t err;
    err = hipFuncSetAttribute((const void*)chunk_intra_kernel<E, DK, DV>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)LI::TOTAL);
    if (err != hipSuccess) return err;
    err = hipFuncSetAttribute((const void*)chunk_inter_kernel<E, DK, DV, TV>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)LX::TOTAL);
    if (err != hipSuccess) return err;
    unsigned char* ws = (unsigned char*)a.workspace;
    hipLaunchKernelGGL((chunk_intra_kernel<E, DK, DV>), dim3(NC, a.H, a.B), dim3(256), LI::TOTAL, st,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta,
                       a.g_min, a.T, a.H, NC, ws);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((chunk_inter_kernel<E, DK, DV, TV>), dim3(DV / TV, a.H, a.B), dim3(256), LX::TOTAL, st,
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
