// seg.hip -- kda_chunk_fwd on bf16 tokens: fused segment kernels.
//
// Same chunk form as the fp32 path (Kimi Linear tech report, section 3.1 and
// appendix B, Propositions 1-2, Eqs. 16-19; beta_r scales the whole
// right-hand side of Eqs. 17 and 19):
//   V_new = U - W S,  O = (Q e^G) S + M V_new,  S' = Diag(e^{G_C}) S + (K e^{G_C-G})^T V_new.
// Here the per-chunk products (W, U, M, Q e^G, K e^{G_C-G}, e^{G_C}) never
// leave the chip: one workgroup of 512 threads walks a segment of chunks of
// one (b, h) chain, computes each chunk's products into LDS from the raw
// tokens, and advances a d_k x N fp32 state held in MFMA accumulators.
//
//  * EXPAND  the state starts from the given entry state; the outputs O are
//            written; the state is S.
//  * COMPOSE the state is [P | R] (d_k x (d_k + d_v)) starting from [I | 0]:
//            the segment's affine map S_end = P S_start + R, with
//            P = prod_n (Diag(e^{G_C}) - K~_n^T W_n) and R the state reached
//            from S_start = 0.  A scan over segments then gives every
//            segment's entry state, and EXPAND runs all segments in parallel.
//
// The first segment of a chain starts from s0 and the last one's transition
// only matters for the final state, so the split plan (pipe_first_kernel,
// pipe_last_kernel) expands those two directly, each beside the compose or
// the light expand of the middle segments: a fifth of the chunks at the 32k
// prefill shape then run once instead of twice.
//
// State in registers.  Each chain wave owns 16-column tiles of the state.  A
// 16x16x32 bf16 MFMA reads operand B as (column l%16, contraction indices
// 8(l/16)..+7) and leaves its result as (column l%16, rows 4(l/16)+e).  Two
// vertically adjacent accumulator tiles therefore hold, in each lane, exactly
// the eight values of a B fragment, up to an order of the contraction index
// inside each 32-block.  That order is fixed once (pcol below), and every
// LDS operand that is contracted against accumulator-held data (K e^G and
// Q e^G against the state; T' against Z; M against V_new; (K e^{G_C-G})^T
// against V_new) is stored with its contraction columns in the same order.
// So Z = V - K e^G S, V_new = T' Z (which is U - W S, with
// T' = (I + A)^{-1} diag(beta)), the outputs and the state update read only
// the shared per-chunk operands from LDS; the state, Z and V_new never
// leave the registers of the wave that owns them.
//
// Overflow handling of the decay factors is that of the fp32 path: A and M
// per 16x16 block pair with reference rows m(R) = 16R + 7, decay exponents in
// log2 units so that every factor is one v_exp_f32, and the cross-block
// factor e^{G_m(R) - G_m(I)} applied as its square root twice (it spans 16
// or more rows and alone could underflow next to a key factor of 2^93).
//
// Two kernels walk the segments.  pipe_kernel (d_k = d_v = 128) splits the
// waves into state waves, which advance the state, and gate waves, which
// prepare the next chunk, so that the MFMA-bound step and the VALU-bound gate
// run side by side on every SIMD.  seg_kernel (every width) runs all phases
// on all waves one after the other; it serves d_k or d_v = 64.
#include <stdlib.h>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace segk {

constexpr int C = 64;       // chunk length
constexpr int SUB = 16;     // block size of A, M and the triangular solve
constexpr int NTH = 512;    // threads per workgroup (8 waves)
constexpr float LOG2E = 1.4426950408889634f;
enum { COMPOSE = 0, EXPAND = 1, EXPAND_LITE = 2 };

constexpr size_t a16(size_t x) { return (x + 15) / 16 * 16; }
constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }

// Storage position of contraction index x: inside each block of 32,
// x = 16 h + 4 g + j is stored at 8 g + 4 h + j, so lane group g of a
// fragment load (8 consecutive stored elements) gets rows 4g..4g+3 of two
// vertically adjacent 16-row accumulator tiles.
__host__ __device__ constexpr int pcol(int x) {
    return (x & ~31) | ((x & 12) << 1) | ((x & 16) >> 2) | (x & 3);
}

// LDS layout (byte offsets) of one workgroup.
template <int DK, int DV, int MODE>
struct Lay {
    static constexpr bool EXP = MODE == EXPAND;
    static constexpr int CP = DK / 2;            // key-channel pairs
    static constexpr int NPART = NTH / CP;       // row parts (8 or 16)
    static constexpr int RP = C / NPART;         // rows per thread (8 or 4)
    static constexpr int CPV = DV / 2;
    static constexpr int RPV = C / (NTH / CPV);
    static constexpr int LDK = DK + 8;           // (C x DK) bf16 tiles
    static constexpr int LC = C + 8;             // (d x C) bf16 tiles
    static constexpr int LB = SUB + 8;           // 16x16 bf16 operand blocks
    static constexpr int BS = SUB * SUB + 16;    // fp32 diagonal block stride (words)
    static constexpr size_t TILE = (size_t)C * LDK * 2;
    static constexpr size_t OFF_KL = 0;                                    // KL, then T' [C][LC] pcol
    static constexpr size_t OFF_TP = OFF_KL;
    static constexpr size_t OFF_KR = TILE;                                 // KR
    static constexpr size_t OFF_QL = OFF_KR + TILE;                        // QL (EXPAND)
    static constexpr size_t OFF_KG = OFF_QL + (EXP ? TILE : 0);            // -k e^G [C][LDK] pcol
    static constexpr size_t OFF_RV = OFF_KG + TILE;                        // v^T [DV][LC]
    static constexpr size_t OFF_KGT = OFF_RV + a16((size_t)DV * LC * 2);   // K~^T [DK][LC] pcol
    static constexpr size_t OFF_QG = OFF_KGT + a16((size_t)DK * LC * 2);   // q e^G [C][LDK] pcol
    static constexpr size_t OFF_M = OFF_QG + (EXP ? TILE : 0);             // M [C][LC] pcol
    static constexpr size_t OFF_AS = OFF_M + (EXP ? a16((size_t)C * LC * 2) : 0);   // diag A blocks fp32
    static constexpr size_t OFF_AB = OFF_AS + (size_t)4 * BS * 4;          // -A off-diag blocks bf16
    static constexpr size_t OFF_DB = OFF_AB + a16((size_t)6 * SUB * LB * 2);   // (I+A_RR)^{-1} bf16
    static constexpr size_t OFF_EGC = OFF_DB + a16((size_t)4 * SUB * LB * 2);
    static constexpr size_t OFF_DSC = OFF_EGC + (size_t)DK * 4;            // [6][DK] block factors
    static constexpr size_t OFF_CAR = OFF_DSC + 6 * (size_t)DK * 4;        // [NPART][DK] part sums
    static constexpr size_t OFF_BET = OFF_CAR + (size_t)NPART * DK * 4;
    static constexpr size_t LDS = OFF_BET + C * 4;
    static_assert(RP % 4 == 0 && RPV % 4 == 0 && 16 % RP == 0, "intra tiling");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// One chunk's raw tokens, as this thread loads them (register prefetch).
template <int DK, int DV, int MODE>
struct In {
    typedef Lay<DK, DV, MODE> L;
    bf16x2 z[L::RP], k[L::RP], q[L::EXP ? L::RP : 1], v[L::RPV];
    bf16 beta;
};

// Loads are unconditional at clamped rows (always in bounds): a load under a
// branch makes the wait-count insertion assume the no-load path.
template <int DK, int DV, int MODE>
__device__ __forceinline__ void fetch_zkq(In<DK, DV, MODE>& r, const bf16* __restrict__ q,
                                          const bf16* __restrict__ k, const bf16* __restrict__ z,
                                          const bf16* __restrict__ beta, size_t row0, int valid, int H) {
    typedef Lay<DK, DV, MODE> L;
    const int tid = threadIdx.x;
    const int c0 = 2 * (tid % L::CP), r0 = (L::CP == 64 ? wave_id() : tid / L::CP) * L::RP;
    const int last = valid - 1, rs = H * DK;
    const bf16* zb = z + row0 * DK;
    const bf16* kb = k + row0 * DK;
    const bf16* qb = q + row0 * DK;
#pragma unroll
    for (int i = 0; i < L::RP; ++i) {
        // row pointer (wave-uniform when a wave spans all channels) + lane offset
        const size_t ro = (size_t)min(r0 + i, last) * rs;
        r.z[i] = load2<bf16>(zb + ro + c0);
        r.k[i] = load2<bf16>(kb + ro + c0);
        if constexpr (L::EXP) r.q[i] = load2<bf16>(qb + ro + c0);
    }
    r.beta = beta[row0 + (size_t)min(tid & (C - 1), last) * H];
}

template <int DK, int DV, int MODE>
__device__ __forceinline__ void fetch_v(In<DK, DV, MODE>& r, const bf16* __restrict__ v, size_t row0, int valid,
                                        int H) {
    typedef Lay<DK, DV, MODE> L;
    const int tid = threadIdx.x;
    const int cv0 = 2 * (tid % L::CPV), rv0 = (L::CPV == 64 ? wave_id() : tid / L::CPV) * L::RPV;
    const bf16* vb = v + row0 * DV;
#pragma unroll
    for (int i = 0; i < L::RPV; ++i) r.v[i] = load2<bf16>(vb + (size_t)min(rv0 + i, valid - 1) * (H * DV) + cv0);
}

// Block pairs (R, I), I <= R, of A and M per wave: the diagonal pairs (no
// cross-block factor) two to a wave.
__constant__ int kSegPairs[8][2][2] = {{{0, 0}, {3, 3}}, {{1, 1}, {2, 2}}, {{1, 0}, {-1, -1}}, {{2, 0}, {-1, -1}},
                                       {{2, 1}, {-1, -1}}, {{3, 0}, {-1, -1}}, {{3, 1}, {-1, -1}}, {{3, 2}, {-1, -1}}};

__device__ __forceinline__ void store4p(bf16* p, float a, float b, float c, float d) {
    store4<bf16>(p, f32x4{a, b, c, d});
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
// 16x16x16 bf16 MFMA: A (row l%16, k 4(l/16)..+3), B (col l%16, same k), C as usual
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                     0, 0);
}
__device__ __forceinline__ bf16x4 to_bf4(f32x4 v) {
    return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// Phase 1 arithmetic on the thread's RP rows of channels c0, c0+1: the gate in
// log2 units and its chunk-local running sum; rows at or past `valid` (only
// in a ragged last chunk) act as identity tokens (g = 0, k = q = 0).
template <bool FULL, int RP, bool EXP>
__device__ __forceinline__ void gate_scan(const bf16x2 (&zr)[RP], const bf16x2 (&kr)[RP],
                                          const bf16x2 (&qr)[EXP ? RP : 1], float kg2, int r0, int valid,
                                          float (&G)[RP][2], float (&kv)[RP][2], float (&qv)[EXP ? RP : 1][2]) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const bool ok = FULL || r0 + i < valid;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float g2 = kg2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * (float)zr[i][j]));
            G[i][j] = ok ? g2 : 0.f;
            kv[i][j] = ok ? (float)kr[i][j] : 0.f;
            if constexpr (EXP) qv[i][j] = ok ? (float)qr[i][j] : 0.f;
        }
        s0 += G[i][0];
        s1 += G[i][1];
        G[i][0] = s0;
        G[i][1] = s1;
    }
}

__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = (bf16)a[i];
        r[i + 4] = (bf16)b[i];
    }
    return r;
}

// ---------------------------------------------------------------------------
// One chunk of the recurrence for one chain wave owning NTW state column
// tiles.  Rows of the state in this lane: 16 rt + 4 (l/16) + e; columns
// col0 + 16 ct + l%16.  With hasu false the value input is zero (the P part
// of COMPOSE).  EXPAND writes the chunk's outputs o[token][ocol0 + ...].
// ---------------------------------------------------------------------------
template <int DK, int DV, int MODE, int NTW, class L = Lay<DK, DV, MODE>>
__device__ __forceinline__ void chain_step(f32x4 (&xs)[DK / 16][NTW], bool hasu, int ucol0, const unsigned char* smem,
                                           bf16* __restrict__ orow0, int valid, size_t ostride) {
    typedef Mfma<bf16> MF;
    constexpr int NKD = DK / 32;
    const int l = lane_id(), g = l >> 4, c = l & 15;
    const bf16* VT = reinterpret_cast<const bf16*>(smem + L::OFF_RV);
    const bf16* Tp = reinterpret_cast<const bf16*>(smem + L::OFF_TP);
    const bf16* KGT = reinterpret_cast<const bf16*>(smem + L::OFF_KGT);
    const bf16* KGn = reinterpret_cast<const bf16*>(smem + L::OFF_KG);
    const bf16* QG = reinterpret_cast<const bf16*>(smem + L::OFF_QG);
    const bf16* Ms = reinterpret_cast<const bf16*>(smem + L::OFF_M);
    const float* egc = reinterpret_cast<const float*>(smem + L::OFF_EGC);

    // Z = V - (K e^G) S (rows 16 yt + 4g + e) and, for EXPAND, the S part of
    // O^T = S^T (Q e^G)^T + V_new^T M^T; one 32-row block of S at a time.
    // Operand fragments are loaded one block ahead of their MFMAs.
    f32x4 y[4][NTW];
#pragma unroll
    for (int yt = 0; yt < 4; ++yt)
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct)
            y[yt][ct] = hasu ? load4<bf16>(VT + (ucol0 + ct * 16 + c) * L::LC + yt * 16 + 4 * g) : zero4();
    f32x4 ov[L::EXP ? 4 : 1][NTW];
    if constexpr (L::EXP) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot)
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) ov[ot][ct] = zero4();
    }
    MF::frag wf[2][4], qf[2][L::EXP ? 4 : 1];
#pragma unroll
    for (int yt = 0; yt < 4; ++yt) wf[0][yt] = load_frag<bf16>(KGn, L::LDK, yt * 16, 0);
    if constexpr (L::EXP) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) qf[0][ot] = load_frag<bf16>(QG, L::LDK, ot * 16, 0);
    }
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) {
        const int cur = kb & 1, nxt = cur ^ 1;
        if (kb + 1 < NKD) {
#pragma unroll
            for (int yt = 0; yt < 4; ++yt) wf[nxt][yt] = load_frag<bf16>(KGn, L::LDK, yt * 16, (kb + 1) * 32);
            if constexpr (L::EXP) {
#pragma unroll
                for (int ot = 0; ot < 4; ++ot) qf[nxt][ot] = load_frag<bf16>(QG, L::LDK, ot * 16, (kb + 1) * 32);
            }
        }
        bf16x8 xb[NTW];
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct) xb[ct] = pack8(xs[2 * kb][ct], xs[2 * kb + 1][ct]);
#pragma unroll
        for (int yt = 0; yt < 4; ++yt)
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) y[yt][ct] = MF::mma(wf[cur][yt], xb[ct], y[yt][ct]);
        if constexpr (L::EXP) {
#pragma unroll
            for (int ot = 0; ot < 4; ++ot)
#pragma unroll
                for (int ct = 0; ct < NTW; ++ct) ov[ot][ct] = MF::mma(xb[ct], qf[cur][ot], ov[ot][ct]);
        }
    }
    // next operands: the first K~^T row block and e^{G_C} (and M for EXPAND)
    MF::frag kf[2][2];
    f32x4 dv[2];
    kf[0][0] = load_frag<bf16>(KGT, L::LC, 0, 0);
    kf[0][1] = load_frag<bf16>(KGT, L::LC, 0, 32);
    dv[0] = *reinterpret_cast<const f32x4*>(egc + 4 * g);
    MF::frag mf[L::EXP ? 4 : 1][2];
    if constexpr (L::EXP) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) {
            mf[ot][0] = load_frag<bf16>(Ms, L::LC, ot * 16, 0);
            mf[ot][1] = load_frag<bf16>(Ms, L::LC, ot * 16, 32);
        }
    }
    // V_new = T' Z with T' = (I + A)^{-1} diag(beta)
    bf16x8 yb[2][NTW];
    {
        bf16x8 zb[2][NTW];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) zb[kb][ct] = pack8(y[2 * kb][ct], y[2 * kb + 1][ct]);
#pragma unroll
        for (int yt = 0; yt < 4; ++yt) {
            const MF::frag t0 = load_frag<bf16>(Tp, L::LC, yt * 16, 0);
            const MF::frag t1 = load_frag<bf16>(Tp, L::LC, yt * 16, 32);
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) {
                y[yt][ct] = MF::mma(t0, zb[0][ct], zero4());
                y[yt][ct] = MF::mma(t1, zb[1][ct], y[yt][ct]);
            }
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct) yb[kb][ct] = pack8(y[2 * kb][ct], y[2 * kb + 1][ct]);

    if constexpr (L::EXP) {
        // lane holds O[16 ot + c][col0 + 16 ct + 4g + e]
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) {
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) {
                ov[ot][ct] = MF::mma(yb[0][ct], mf[ot][0], ov[ot][ct]);
                ov[ot][ct] = MF::mma(yb[1][ct], mf[ot][1], ov[ot][ct]);
            }
            if (ot * 16 + c < valid) {
                bf16* orow = orow0 + (size_t)(ot * 16 + c) * ostride + 4 * g;
#pragma unroll
                for (int ct = 0; ct < NTW; ++ct) store4<bf16>(orow + ct * 16, ov[ot][ct]);
            }
        }
    }

    // S <- Diag(e^{G_C}) S + K~^T V_new
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt) {
        const int cur = rt & 1, nxt = cur ^ 1;
        if (rt + 1 < DK / 16) {
            kf[nxt][0] = load_frag<bf16>(KGT, L::LC, (rt + 1) * 16, 0);
            kf[nxt][1] = load_frag<bf16>(KGT, L::LC, (rt + 1) * 16, 32);
            dv[nxt] = *reinterpret_cast<const f32x4*>(egc + (rt + 1) * 16 + 4 * g);
        }
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct) {
            xs[rt][ct] *= dv[cur];
            xs[rt][ct] = MF::mma(kf[cur][0], yb[0][ct], xs[rt][ct]);
            xs[rt][ct] = MF::mma(kf[cur][1], yb[1][ct], xs[rt][ct]);
        }
    }
}

// Chain waves and tiles per wave.  EXPAND: the DV/16 value tiles; COMPOSE:
// the DK/16 tiles of P followed by the DV/16 tiles of R (a wave's tiles are
// all P or all R since DK/16 is even).
template <int DK, int DV, int MODE>
struct Tiles {
    static constexpr int N = MODE == EXPAND ? DV / 16 : (DK + DV) / 16;
    static constexpr int NTW = N > 8 ? 2 : 1;
    static constexpr int NWAVES = (N + NTW - 1) / NTW;
    static_assert(NWAVES <= 8, "chain waves");
};

// Right-looking substitution steps for columns I0..I1-1 of a 16x16
// strictly lower block stored transposed (at[i * 16 + r] = A_ri):
// x_r -= A_ri x_i for r > i.
template <int I0, int I1>
__device__ __forceinline__ void inv_batch(const float* at, float (&x)[SUB]) {
    f32x4 av[I1 - I0][4];
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int r4 = (i + 1) / 4; r4 < 4; ++r4) av[i - I0][r4] = *reinterpret_cast<const f32x4*>(at + i * SUB + 4 * r4);
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int r4 = (i + 1) / 4; r4 < 4; ++r4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * r4 + e > i) x[4 * r4 + e] -= av[i - I0][r4][e] * x[i];
}

// ---------------------------------------------------------------------------
// The chunk's own products, from its tokens in `in`, into LDS.  On return
// (after a barrier) LDS holds T' = (I + A)^{-1} diag(beta), -K e^G, V^T,
// K~^T, e^{G_C} and, for EXPAND, Q e^G and M.  `in` is refilled with chunk
// `nx` once its values are consumed.
//
//  1  gate, chunk-local running sum of the log2 decay per channel; carries
//     between row parts through LDS                                  | barrier
//  2  block reference values G_m(R) from the carries; the decay-scaled
//     operands k e^{G_r - G_m(R)}, k e^{G_m(R) - G_r}, q e^{G_r - G_m(R)},
//     -k e^G, v^T, (k e^{G_C - G})^T, q e^G and the cross-block factors
//     e^{G_m(R) - G_m(I)}                                            | barrier
//  3  A (and M) per 16x16 block pair on MFMA; the waves holding the
//     diagonal blocks invert them, beta folded in: D'_R             | barrier
//  4  T' by block forward substitution on the identity's columns; the
//     chain then forms V_new = T' (V - K e^G S), which is U - W S    | barrier
// ---------------------------------------------------------------------------
template <int DK, int DV, int MODE>
__device__ __forceinline__ void intra(In<DK, DV, MODE>& in, int valid, float g_min, unsigned char* smem,
                                      const bf16* __restrict__ q, const bf16* __restrict__ k,
                                      const bf16* __restrict__ v, const bf16* __restrict__ z,
                                      const bf16* __restrict__ beta, size_t nx_row0, int nx_valid, int H) {
    typedef Lay<DK, DV, MODE> L;
    typedef Mfma<bf16> MF;
    constexpr bool EXP = L::EXP;
    constexpr int LDK = L::LDK, LC = L::LC, RP = L::RP, RPV = L::RPV, LB = L::LB, BS = L::BS;

    bf16* KL = reinterpret_cast<bf16*>(smem + L::OFF_KL);   // [C][LDK] k e^{G_r - G_m(R)}
    bf16* KR = reinterpret_cast<bf16*>(smem + L::OFF_KR);   // [C][LDK] k e^{G_m(R) - G_r}
    bf16* QL = reinterpret_cast<bf16*>(smem + L::OFF_QL);   // [C][LDK] q e^{G_r - G_m(R)}
    bf16* Tp = reinterpret_cast<bf16*>(smem + L::OFF_KL);   // [C][LC] T' = (I+A)^{-1} diag(beta), pcol (phase 4 on)
    bf16* KGn = reinterpret_cast<bf16*>(smem + L::OFF_KG);  // [C][LDK] -k e^G, pcol
    bf16* RV = reinterpret_cast<bf16*>(smem + L::OFF_RV);   // [DV][LC]
    bf16* KGT = reinterpret_cast<bf16*>(smem + L::OFF_KGT); // [DK][LC] pcol
    bf16* QG = reinterpret_cast<bf16*>(smem + L::OFF_QG);   // [C][LDK] pcol
    bf16* Ms = reinterpret_cast<bf16*>(smem + L::OFF_M);    // [C][LC] pcol
    float* As = reinterpret_cast<float*>(smem + L::OFF_AS); // [4][BS] diagonal blocks, row stride 16
    bf16* Ab = reinterpret_cast<bf16*>(smem + L::OFF_AB);   // [6][16][LB] -A_RJ
    bf16* Db = reinterpret_cast<bf16*>(smem + L::OFF_DB);   // [4][16][LB] (I + A_RR)^{-1}
    float* egc = reinterpret_cast<float*>(smem + L::OFF_EGC);
    float* dsc = reinterpret_cast<float*>(smem + L::OFF_DSC);   // [6][DK] e^{(G_m(R) - G_m(I)) / 2}
    float* car = reinterpret_cast<float*>(smem + L::OFF_CAR);   // [NPART][DK]
    float* bet = reinterpret_cast<float*>(smem + L::OFF_BET);   // [C]

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    __builtin_assume(w >= 0 && w < NTH / 64);
    // row part of this thread: one per wave when a wave spans all key channels
    const int part = L::CP == 64 ? w : tid / L::CP;
    const int c0 = 2 * (tid % L::CP), r0 = part * RP;
    const int cv0 = 2 * (tid % L::CPV), rv0 = (tid / L::CPV) * RPV;

    // ---- phase 1
    if (tid < C) bet[tid] = tid < valid ? (float)in.beta : 0.f;
    const float kg2 = g_min * LOG2E;
    float G[RP][2], kv[RP][2], qv[EXP ? RP : 1][2];
    if (valid == C)
        gate_scan<true, RP, EXP>(in.z, in.k, in.q, kg2, r0, valid, G, kv, qv);
    else
        gate_scan<false, RP, EXP>(in.z, in.k, in.q, kg2, r0, valid, G, kv, qv);
    fetch_zkq<DK, DV, MODE>(in, q, k, z, beta, nx_row0, nx_valid, H);
    car[part * DK + c0] = G[RP - 1][0];
    car[part * DK + c0 + 1] = G[RP - 1][1];
    __syncthreads();

    // ---- phase 2
    {
        // carry into this part, block reference values G_m(R') (row 16R'+7
        // closes part (16R'+8)/RP - 1) and the chunk total G_C
        float cr[2] = {0.f, 0.f}, gC[2] = {0.f, 0.f}, gm[4][2];
#pragma unroll
        for (int p = 0; p < L::NPART; ++p)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float t = car[p * DK + c0 + j];
                if (p < part) cr[j] += t;
                gC[j] += t;
#pragma unroll
                for (int R = 0; R < 4; ++R)
                    if (p == (16 * R + 8) / RP - 1) gm[R][j] = gC[j];
            }
        const int R = r0 >> 4;
        float gmR[2], eGm[2], eCGm[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            gmR[j] = R == 0 ? gm[0][j] : R == 1 ? gm[1][j] : R == 2 ? gm[2][j] : gm[3][j];
            eGm[j] = __builtin_amdgcn_exp2f(gmR[j]);
            eCGm[j] = __builtin_amdgcn_exp2f(gC[j] - gmR[j]);
        }
        if (part == 0) {
            egc[c0] = __builtin_amdgcn_exp2f(gC[0]);
            egc[c0 + 1] = __builtin_amdgcn_exp2f(gC[1]);
        }
        if (part < 6) {
            // pair index p = R'(R'-1)/2 + I', I' < R'
            const int Rp = part < 1 ? 1 : (part < 3 ? 2 : 3);
            const int Ip = part - Rp * (Rp - 1) / 2;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float a = gm[0][j], b = gm[0][j];
#pragma unroll
                for (int t = 1; t < 4; ++t) {
                    if (Rp == t) a = gm[t][j];
                    if (Ip == t) b = gm[t][j];
                }
                dsc[part * DK + c0 + j] = __builtin_amdgcn_exp2f(0.5f * (a - b));   // applied twice
            }
        }
        float kg[2][RP];
        const float off[2] = {cr[0] - gmR[0], cr[1] - gmR[1]};   // row r: G2_r - G2_m(R) = G[i] + off
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
            float kl[2], kR[2], ql[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float el = G[i][j] + off[j];
                const float left = __builtin_amdgcn_exp2f(el), right = __builtin_amdgcn_exp2f(-el);
                kl[j] = kv[i][j] * left;
                kR[j] = kv[i][j] * right;
                if constexpr (EXP) ql[j] = qv[i][j] * left;
                kg[j][i] = kR[j] * eCGm[j];
            }
            store2<bf16>(KL + r * LDK + c0, kl[0], kl[1]);
            store2<bf16>(KR + r * LDK + c0, kR[0], kR[1]);
            store2<bf16>(KGn + r * LDK + pcol(c0), -kl[0] * eGm[0], -kl[1] * eGm[1]);
            if constexpr (EXP) {
                store2<bf16>(QL + r * LDK + c0, ql[0], ql[1]);
                store2<bf16>(QG + r * LDK + pcol(c0), ql[0] * eGm[0], ql[1] * eGm[1]);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < RP; i += 4) {
                store4p(KGT + (c0 + j) * LC + pcol(r0 + i), kg[j][i], kg[j][i + 1], kg[j][i + 2], kg[j][i + 3]);
            }
        // V^T as loaded (rows past the end are multiplied by beta = 0 through
        // the beta-scaled diagonal inverses, so their values do not matter)
#pragma unroll
        for (int i = 0; i < RPV; i += 4)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                *reinterpret_cast<bf16x4*>(RV + (cv0 + j) * LC + rv0 + i) =
                    bf16x4{in.v[i][j], in.v[i + 1][j], in.v[i + 2][j], in.v[i + 3][j]};
        fetch_v<DK, DV, MODE>(in, v, nx_row0, nx_valid, H);
    }
    __syncthreads();

    // ---- phase 3: A (and M) per 16x16 block pair, computed transposed so each
    //      lane holds four consecutive key indices i of one row r
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int R = kSegPairs[w][j][0], I = kSegPairs[w][j][1];
        if (R < 0) break;
        f32x4 accA = zero4(), accM = zero4();
        const float* dv = dsc + (R * (R - 1) / 2 + I) * DK;
#pragma unroll
        for (int kk = 0; kk < DK; kk += MF::KSTEP) {
            MF::frag ak = load_frag<bf16>(KR, LDK, I * SUB, kk);
            if (I < R) {
                float t[MF::KPL];
                MF::to_floats(ak, t);
                const int cc = kk + (l >> 4) * MF::KPL;
#pragma unroll
                for (int jj = 0; jj < MF::KPL; ++jj) t[jj] = (t[jj] * dv[cc + jj]) * dv[cc + jj];
                ak = MF::from_floats(t);
            }
            accA = MF::mma(ak, load_frag<bf16>(KL, LDK, R * SUB, kk), accA);
            if constexpr (EXP) accM = MF::mma(ak, load_frag<bf16>(QL, LDK, R * SUB, kk), accM);
        }
        const int rr = l & 15, r = R * SUB + rr;
        const int ii = 4 * (l >> 4), i0 = I * SUB + ii;
        if (I == R) {
            // beta_r A_ri, strictly lower, stored transposed: As[R][i][r]
            const float br = bet[r];
#pragma unroll
            for (int e = 0; e < 4; ++e) As[R * BS + (ii + e) * SUB + rr] = (ii + e < rr) ? br * accA[e] : 0.f;
        } else {
            // -A~_RI without the row factor beta_r (it is folded into the inverses)
            store4p(Ab + ((R * (R - 1) / 2 + I) * SUB + rr) * LB + ii, -accA[0], -accA[1], -accA[2], -accA[3]);
        }
        if constexpr (EXP) {
            float mv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) mv[e] = (i0 + e <= r) ? accM[e] : 0.f;
            store4p(Ms + r * LC + pcol(i0), mv[0], mv[1], mv[2], mv[3]);
        }
    }
    if constexpr (EXP) {
        // strictly upper blocks of M are zero: waves 2..7 one block each
        if (w >= 2) {
            const int p = w - 2;
            const int R = p < 3 ? 0 : (p < 5 ? 1 : 2);
            const int I = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
            store4p(Ms + (R * SUB + (l & 15)) * LC + pcol(I * SUB + 4 * (l >> 4)), 0.f, 0.f, 0.f, 0.f);
        }
    }
    // ---- phase 4a: waves 0 and 1 invert the two diagonal blocks they have
    //      just formed, D'_b = (I + beta_b A~_bb)^{-1} diag(beta_b), lane =
    //      (block, column), by right-looking substitution down the column
    if (w < 2) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // this wave's As stores
        const int b = kSegPairs[w][(l >> 4) & 1][0], col = l & 15;
        const float* at = As + b * BS;       // at[i * 16 + r] = beta_r A~_ri
        float x[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) x[r] = (r == col) ? 1.f : 0.f;
        // columns of A in three batches; a batch's 4-row pieces below the
        // diagonal are all loaded before they are used
        inv_batch<0, 3>(at, x);
        inv_batch<3, 7>(at, x);
        inv_batch<7, 15>(at, x);
        if (l < 32) {
            const float bc = bet[b * SUB + col];
            bf16* d = Db + b * SUB * LB + col;
#pragma unroll
            for (int r = 0; r < SUB; ++r) d[r * LB] = (bf16)(x[r] * bc);
        }
    }
    __syncthreads();

    // ---- phase 4: T' = (I + A)^{-1} diag(beta) by block forward substitution
    //      on the columns of the identity.  Wave w < 4 owns column block w:
    //      X_R = D'_R (E_R - sum_{J<R} A~_RJ X_J) with E the identity, so
    //      X_R = 0 above the diagonal and X_w = D'_w.
    if (w < 4) {
        const int g = l >> 4, c = l & 15;
        bf16x4 ab[6], db[4];
#pragma unroll
        for (int p = 0; p < 6; ++p) ab[p] = *reinterpret_cast<const bf16x4*>(Ab + (p * SUB + c) * LB + 4 * g);
#pragma unroll
        for (int R = 0; R < 4; ++R) db[R] = *reinterpret_cast<const bf16x4*>(Db + (R * SUB + c) * LB + 4 * g);
        f32x4 eye;
#pragma unroll
        for (int e = 0; e < 4; ++e) eye[e] = (4 * g + e == c) ? 1.f : 0.f;
        bf16x4 xb[4];
        bf16* tcol = Tp + 4 * g * LC + pcol(16 * w + c);
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4 x = zero4();
            if (R >= w) {
                f32x4 acc = (R == w) ? eye : zero4();
#pragma unroll
                for (int J = 0; J < R; ++J)
                    if (J >= w) acc = mma16(ab[R * (R - 1) / 2 + J], xb[J], acc);
                x = mma16(db[R], to_bf4(acc), zero4());
            }
            xb[R] = to_bf4(x);
#pragma unroll
            for (int e = 0; e < 4; ++e) tcol[(R * SUB + e) * LC] = xb[R][e];
        }
    }
    __syncthreads();
}

// Grid: one workgroup per (segment, chain), chain index fastest.  Segment s
// covers chunks [s L, min(s L + L, NC)).
//   EXPAND : xin  entry states [nseg][B*H][DK][DV] (NULL = zeros);
//            xo0  final state [B*H][DK][DV] (NULL = skip; used when nseg == 1).
//   COMPOSE: xo0  P [nseg][B*H][DK][DK],  xo1  R [nseg][B*H][DK][DV].
template <int DK, int DV, int MODE>
__global__ __launch_bounds__(NTH) void seg_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                  const bf16* __restrict__ v, const bf16* __restrict__ z,
                                                  const bf16* __restrict__ beta, float g_min, int T, int H, int NC,
                                                  int L, int nchain, const float* __restrict__ xin,
                                                  float* __restrict__ xo0, float* __restrict__ xo1,
                                                  bf16* __restrict__ o) {
    typedef Tiles<DK, DV, MODE> TL;
    constexpr int NTW = TL::NTW;
    extern __shared__ __align__(16) unsigned char smem[];
    const int seg = blockIdx.x / nchain;
    const size_t bh = blockIdx.x % nchain;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int l = lane_id(), w = wave_id();
    __builtin_assume(w >= 0 && w < NTH / 64);
    const int n0 = seg * L, n1 = min(NC, n0 + L);
    const int t0w = w * NTW;                    // first tile of this wave
    const bool chain_wave = w < TL::NWAVES;
    const bool ptile = MODE == COMPOSE && t0w < DK / 16;
    const int col0 = 16 * t0w - (MODE == COMPOSE && !ptile ? DK : 0);   // first column in P, R or S
    const int NX = (MODE == COMPOSE && ptile) ? DK : DV;                // columns of this wave's matrix

    f32x4 xs[DK / 16][NTW];
    const size_t xblk = ((size_t)seg * nchain + bh) * DK;
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = rt * 16 + 4 * (l >> 4) + e, col = col0 + ct * 16 + (l & 15);
                float x = 0.f;
                if constexpr (MODE == EXPAND) x = (xin && chain_wave) ? xin[(xblk + row) * DV + col] : 0.f;
                if constexpr (MODE == COMPOSE) x = (ptile && row == col) ? 1.f : 0.f;
                xs[rt][ct][e] = x;
            }

    In<DK, DV, MODE> in;
    {
        const size_t row0 = ((size_t)b * T + (size_t)n0 * C) * H + h;
        const int valid = min(C, T - n0 * C);
        fetch_zkq<DK, DV, MODE>(in, q, k, z, beta, row0, valid, H);
        fetch_v<DK, DV, MODE>(in, v, row0, valid, H);
    }
    const size_t ostride = (size_t)H * DV;
    const bool hasu = MODE == EXPAND || !ptile;
    auto orow = [&](int n) { return o + (((size_t)b * T + (size_t)n * C) * H + h) * DV + col0; };
    for (int n = n0; n < n1; ++n) {
        const int valid = min(C, T - n * C);
        const int nn = min(n + 1, n1 - 1);      // prefetch target, clamped (unconditional)
        intra<DK, DV, MODE>(in, valid, g_min, smem, q, k, v, z, beta, ((size_t)b * T + (size_t)nn * C) * H + h,
                            min(C, T - nn * C), H);
        // the next chunk's phase 1 writes neither the chain operands nor
        // anything the chain reads: no barrier after the chain step
        if (chain_wave) chain_step<DK, DV, MODE, NTW>(xs, hasu, col0, smem, orow(n), valid, ostride);
    }

    float* xo = MODE == COMPOSE ? (ptile ? xo0 : xo1) : xo0;
    if (chain_wave && xo) {
        const size_t ob = MODE == COMPOSE ? xblk : bh * DK;
#pragma unroll
        for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = rt * 16 + 4 * (l >> 4) + e, col = col0 + ct * 16 + (l & 15);
                    xo[(ob + row) * NX + col] = xs[rt][ct][e];
                }
    }
}

// ---------------------------------------------------------------------------
// Pipelined fused kernel for d_k = d_v = 128.  Waves 0-3 own the state and
// run the recurrence step of chunk m-1 while waves 4-7 compute the gate,
// the decay-scaled operands and the solve of chunk m, so that the MFMA-bound
// step and the VALU-bound gate overlap on every SIMD.  Gate wave 4 + R
// handles rows 16R..16R+15 of a chunk over all key channels.  The block
// reference row 16R+7 lies in its own rows, so the factors
// e^{+-(G_r - G_m(R))}, the diagonal blocks A_RR, M_RR and the inverse of
// I + beta_R A~_RR need nothing from the other waves; block sums and
// references are exchanged through LDS at the first barrier.
//
// Modes: COMPOSE runs the state [P | R] and hands every chunk's T' to the
// expand pass; EXPAND (one segment per chain) forms everything itself;
// EXPAND_LITE reads T' back and forms only M, the step's operands and the
// outputs.
//
// Iteration i, chunk m = n0 + i (COMPOSE, EXPAND):
//  S1  gate waves: gate, block-local running sums, k e^{G-G_m}, k e^{G_m-G}
//                  (and q e^{G-G_m}); block sums and references
//      state waves: recurrence step of chunk m-1 (reads only its operands:
//                  T', -k e^G, v^T, K~^T, e^{G_C} (and q e^G, M))      | barrier
//  S2  gate waves: absolute references; -k e^G, (k e^{G_C-G})^T, e^{G_C},
//                  v^T (and q e^G); A_RR (and M_RR) on MFMA, then
//                  D'_R = (I + beta_R A~_RR)^{-1} diag(beta_R)
//      state waves: the six off-diagonal block pairs of A (and M) with their
//                  cross-block factors e^{G_m(R) - G_m(I)}              | barrier
//  S3  gate waves: T' column blocks (COMPOSE: state waves finish chunk
//                  m-1's state update meanwhile)                        | barrier
// EXPAND_LITE: S1 as above (no k e^{G-G_m}); S2 forms M_RR and the pairs
// of M, the operands, stores T' from the compose pass and the next chunk's
// running sums                                                          | barrier
// State tiles: the expand modes, wave w owns columns 32w..32w+31 of S;
// COMPOSE, waves 0-1 own 64 columns of P and waves 2-3 64 columns of R,
// advanced 32 columns at a time.
// ---------------------------------------------------------------------------
template <int MODE>
struct PLay {
    static constexpr int DK = 128, DV = 128;
    static constexpr bool EXP = MODE != COMPOSE;      // outputs O (and so q, M)
    static constexpr bool LITE = MODE == EXPAND_LITE; // T' read from the compose pass
    static constexpr bool SOLVE = !LITE;              // A, its inverses and T' formed here
    // Row pitches (bf16 elements).  A 16-row fragment read (16 bytes per
    // lane, rows 16 apart in lanes) meets no LDS bank conflict on gfx950 when
    // the pitch is 32 bytes (mod 64) past a multiple of 256; 272- and
    // 144-byte rows cost two passes.  EXPAND has no LDS left for the wider
    // rows and keeps LDK = 136, LT = 72.
    static constexpr bool WIDE = MODE != EXPAND;
    static constexpr int LDK = WIDE ? DK + 16 : DK + 8;   // [C][DK] operands: 288-byte rows
    static constexpr int LT = WIDE ? C + 16 : C + 8;      // T' and M: 160-byte rows
    static constexpr int LC = C + 8, LB = SUB + 8, BS = SUB * SUB + 16;
    static constexpr size_t TILE = (size_t)C * LDK * 2;
    static constexpr size_t CC = a16((size_t)C * LT * 2);                 // one C x C bf16 operand
    static constexpr size_t OFF_TP = 0;                                    // T' [C][LT] pcol
    static constexpr size_t OFF_KL = CC;                                   // [C][LDK] k e^{G_r - G_m(R)}
    static constexpr size_t OFF_KR = OFF_KL + TILE;                        // [C][LDK] k e^{G_m(R) - G_r}
    static constexpr size_t OFF_QL = OFF_KR + TILE;                        // [C][LDK] q e^{G_r - G_m(R)} (outputs)
    static constexpr size_t OFF_KG = OFF_QL + (EXP ? TILE : 0);            // -k e^G [C][LDK] pcol
    static constexpr size_t OFF_RV = OFF_KG + TILE;                        // v^T [DV][LC]
    // K~^T and e^{G_C}: COMPOSE keeps two buffers (by chunk parity), so that
    // chunk m-1's state update can run while chunk m's are written
    static constexpr int NKB = MODE == COMPOSE ? 2 : 1;
    static constexpr size_t KGT_SZ = a16((size_t)DK * LC * 2);
    static constexpr size_t OFF_KGT = OFF_RV + a16((size_t)DV * LC * 2);   // K~^T [DK][LC] pcol
    static constexpr size_t OFF_QG = OFF_KGT + NKB * KGT_SZ;               // q e^G [C][LDK] pcol (outputs)
    static constexpr size_t OFF_M = OFF_QG + (EXP ? TILE : 0);             // M [C][LT] pcol (outputs)
    static constexpr size_t OFF_AS = OFF_M + (EXP ? CC : 0);               // [4][BS] beta A~_RR^T
    static constexpr size_t OFF_AB = OFF_AS + (SOLVE ? (size_t)4 * BS * 4 : 0);             // [6][16][LB] -A~_RI
    static constexpr size_t OFF_DB = OFF_AB + (SOLVE ? a16((size_t)6 * SUB * LB * 2) : 0);  // [4][16][LB] D'_R
    static constexpr size_t OFF_EGC = OFF_DB + (SOLVE ? a16((size_t)4 * SUB * LB * 2) : 0);
    static constexpr size_t OFF_DSC = OFF_EGC + NKB * (size_t)DK * 4;      // [6][DK] e^{(G_m(R) - G_m(I)) / 2}
    static constexpr size_t OFF_TOT = OFF_DSC + 6 * (size_t)DK * 4;        // [4][DK] block sums
    static constexpr size_t OFF_MLOC = OFF_TOT + 4 * (size_t)DK * 4;       // [4][DK] G_m(R) - G_{16R-1}
    static constexpr size_t OFF_BET = OFF_MLOC + 4 * (size_t)DK * 4;
    static constexpr size_t LDS = OFF_BET + C * 4;
    // EXPAND_LITE forms no A, so the KL tile is free: with the output
    // epilogue fused it holds the chunk's outputs O [C][LDK] in bf16
    static constexpr size_t OFF_OT = OFF_KL;
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Per-chunk T' handed from the compose pass to the expand pass: per (chain,
// chunk) one 64 x 64 bf16 matrix, rows of 64 in the LDS column order (pcol),
// 8 KB.
constexpr size_t TM_ELEMS = (size_t)C * C;

// Piece p (16 bytes) of a chunk's T': row p / 8, eighth p % 8 of the row; its
// place in LDS (padded rows of LT).
template <class L>
__device__ __forceinline__ f32x4* tp_lds(unsigned char* smem, int p) {
    return reinterpret_cast<f32x4*>(smem + L::OFF_TP + (size_t)(p >> 3) * L::LT * 2 + (p & 7) * 16);
}

// Recurrence step of the pipelined kernel, first part: V_new = T' Z with
// Z = V - (K e^G) S, left in yb as bf16 B fragments, and for EXPAND the
// outputs O = (Q e^G) S + M V_new.  Same register layouts as chain_step.
// GATED (EXPAND_LITE with the output epilogue fused): the outputs, rounded
// to bf16, go to the staging tile for the epilogue, and to o only when orow0
// is not NULL.
template <int MODE, int NTW, class L, bool GATED = false>
__device__ __forceinline__ void chain_a(const f32x4 (&xs)[8][NTW], bf16x8 (&yb)[2][NTW], bool hasu, int ucol0,
                                        unsigned char* smem, bf16* __restrict__ orow0, int valid,
                                        size_t ostride) {
    typedef Mfma<bf16> MF;
    constexpr bool EXP = L::EXP;
    const int l = lane_id(), g = l >> 4, c = l & 15;
    const bf16* VT = reinterpret_cast<const bf16*>(smem + L::OFF_RV);
    const bf16* Tp = reinterpret_cast<const bf16*>(smem + L::OFF_TP);
    const bf16* KGn = reinterpret_cast<const bf16*>(smem + L::OFF_KG);
    const bf16* QG = reinterpret_cast<const bf16*>(smem + L::OFF_QG);
    const bf16* Ms = reinterpret_cast<const bf16*>(smem + L::OFF_M);
    f32x4 y[4][NTW];
#pragma unroll
    for (int yt = 0; yt < 4; ++yt)
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct)
            y[yt][ct] = hasu ? load4<bf16>(VT + (ucol0 + ct * 16 + c) * L::LC + yt * 16 + 4 * g) : zero4();
    f32x4 ov[EXP ? 4 : 1][NTW];
    if constexpr (EXP) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot)
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) ov[ot][ct] = zero4();
    }
    MF::frag wf[2][4], qf[2][EXP ? 4 : 1];
#pragma unroll
    for (int yt = 0; yt < 4; ++yt) wf[0][yt] = load_frag<bf16>(KGn, L::LDK, yt * 16, 0);
    if constexpr (EXP) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) qf[0][ot] = load_frag<bf16>(QG, L::LDK, ot * 16, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int cur = kb & 1, nxt = cur ^ 1;
        if (kb + 1 < 4) {
#pragma unroll
            for (int yt = 0; yt < 4; ++yt) wf[nxt][yt] = load_frag<bf16>(KGn, L::LDK, yt * 16, (kb + 1) * 32);
            if constexpr (EXP) {
#pragma unroll
                for (int ot = 0; ot < 4; ++ot) qf[nxt][ot] = load_frag<bf16>(QG, L::LDK, ot * 16, (kb + 1) * 32);
            }
        }
        bf16x8 xb[NTW];
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct) xb[ct] = pack8(xs[2 * kb][ct], xs[2 * kb + 1][ct]);
#pragma unroll
        for (int yt = 0; yt < 4; ++yt)
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) y[yt][ct] = MF::mma(wf[cur][yt], xb[ct], y[yt][ct]);
        if constexpr (EXP) {
#pragma unroll
            for (int ot = 0; ot < 4; ++ot)
#pragma unroll
                for (int ct = 0; ct < NTW; ++ct) ov[ot][ct] = MF::mma(xb[ct], qf[cur][ot], ov[ot][ct]);
        }
    }
    MF::frag mf[EXP ? 4 : 1][2];
    if constexpr (EXP) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) {
            mf[ot][0] = load_frag<bf16>(Ms, L::LT, ot * 16, 0);
            mf[ot][1] = load_frag<bf16>(Ms, L::LT, ot * 16, 32);
        }
    }
    {
        bf16x8 zb[2][NTW];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) zb[kb][ct] = pack8(y[2 * kb][ct], y[2 * kb + 1][ct]);
        // T' fragments one row tile ahead
        MF::frag tf[2][2];
        tf[0][0] = load_frag<bf16>(Tp, L::LT, 0, 0);
        tf[0][1] = load_frag<bf16>(Tp, L::LT, 0, 32);
#pragma unroll
        for (int yt = 0; yt < 4; ++yt) {
            const int cur = yt & 1, nxt = cur ^ 1;
            if (yt + 1 < 4) {
                tf[nxt][0] = load_frag<bf16>(Tp, L::LT, (yt + 1) * 16, 0);
                tf[nxt][1] = load_frag<bf16>(Tp, L::LT, (yt + 1) * 16, 32);
            }
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) {
                y[yt][ct] = MF::mma(tf[cur][0], zb[0][ct], zero4());
                y[yt][ct] = MF::mma(tf[cur][1], zb[1][ct], y[yt][ct]);
            }
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct) yb[kb][ct] = pack8(y[2 * kb][ct], y[2 * kb + 1][ct]);
    if constexpr (EXP) {
        // lane holds O[16 ot + c][col0 + 16 ct + 4g + e]
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) {
#pragma unroll
            for (int ct = 0; ct < NTW; ++ct) {
                ov[ot][ct] = MF::mma(yb[0][ct], mf[ot][0], ov[ot][ct]);
                ov[ot][ct] = MF::mma(yb[1][ct], mf[ot][1], ov[ot][ct]);
            }
            if constexpr (GATED) {
                bf16x4 ob[NTW];
#pragma unroll
                for (int ct = 0; ct < NTW; ++ct) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) ob[ct][e] = (bf16)ov[ot][ct][e];
                    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(smem + L::OFF_OT) +
                                               (ot * 16 + c) * L::LDK + ucol0 + ct * 16 + 4 * g) = ob[ct];
                }
                if (orow0 && ot * 16 + c < valid) {
                    int lg = l;
                    asm volatile("" : "+v"(lg));
                    char* orow = reinterpret_cast<char*>(orow0) +
                                 (unsigned)(ot * 16 + (lg & 15)) * ((unsigned)ostride * 2u) + 8u * (unsigned)(lg >> 4);
#pragma unroll
                    for (int ct = 0; ct < NTW; ++ct) *reinterpret_cast<bf16x4*>(orow + ct * 32) = ob[ct];
                }
            } else {
                static_assert(NTW == 2, "the paired stores assume two column tiles");
                // lanes 16 apart swap halves, so that each holds 8 consecutive
                // columns of its row (even l/16: 4g..4g+7, odd: 4g+12..4g+19)
                // and one store covers 64 contiguous bytes per row
                bf16x4 b[2];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) b[ct][e] = (bf16)ov[ot][ct][e];
                // lane-derived values recomputed here, not held across the loop
                int lx = l;
                asm volatile("" : "+v"(lx));
                const bool odd = (lx >> 4) & 1;
                const uint2 send = __builtin_bit_cast(uint2, odd ? b[0] : b[1]);
                const int src = (lx ^ 16) << 2;
                const uint2 recv = {(unsigned)__builtin_amdgcn_ds_bpermute(src, (int)send.x),
                                    (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)send.y)};
                const bf16x4 r = __builtin_bit_cast(bf16x4, recv);
                const bf16x4 lo4 = odd ? r : b[0], hi4 = odd ? b[1] : r;
                const bf16x8 out = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                if (ot * 16 + (lx & 15) < valid)
                    *reinterpret_cast<bf16x8*>(reinterpret_cast<char*>(orow0) +
                                               (unsigned)(ot * 16 + (lx & 15)) * ((unsigned)ostride * 2u) +
                                               8u * (unsigned)(lx >> 4) + (odd ? 24u : 0u)) = out;
            }
        }
    }
}

// Fused output epilogue: y = o / sqrt(mean(o^2) + eps) * sigmoid(gate) over
// the 128 values of each (token, head) row of the chunk, for NP passes of four
// rows from row r0 (lane: row r0 + 4p + l/16, values 8 (l%16) .. +7), from the
// bf16 outputs in the staging tile.  The gate logits come from gate_fetch.
// Addresses: a wave-uniform chunk base plus 32-bit byte offsets, derived
// from the lane inside the loop (not hoisted into registers held across it).
template <int NP>
__device__ __forceinline__ void gate_fetch(bf16x8 (&gk)[6], const bf16* __restrict__ grow0, int r0, int valid,
                                           size_t ostride) {
    int l = lane_id();
    asm volatile("" : "+v"(l));
    const char* gb = reinterpret_cast<const char*>(grow0);
    const unsigned rs = (unsigned)ostride * 2u, lo = 16u * (unsigned)(l & 15);
#pragma unroll
    for (int p = 0; p < NP; ++p)
        gk[p] = *reinterpret_cast<const bf16x8*>(gb + (unsigned)min(r0 + 4 * p + (l >> 4), valid - 1) * rs + lo);
}
template <int NP, class L>
__device__ __forceinline__ void gate_epilogue(const bf16x8 (&gk)[6], const unsigned char* smem, float eps,
                                              bf16* __restrict__ yrow0, int r0, int valid, size_t ostride) {
    int l = lane_id();
    asm volatile("" : "+v"(l));
    const bf16* OT = reinterpret_cast<const bf16*>(smem + L::OFF_OT);
    char* yb = reinterpret_cast<char*>(yrow0);
    const unsigned rs = (unsigned)ostride * 2u;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = r0 + 4 * p + (l >> 4);
        const bf16x8 ob = *reinterpret_cast<const bf16x8*>(OT + r * L::LDK + 8 * (l & 15));
        float x[8], ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x[j] = (float)ob[j];
            ss += x[j] * x[j];
        }
        // sum over the row's 16 lanes (one DPP row): xor 1, xor 2, then the
        // half-row and row mirrors
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0xB1, 0xF, 0xF, false));
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x4E, 0xF, 0xF, false));
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x141, 0xF, 0xF, false));
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x140, 0xF, 0xF, false));
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / 128) + eps);
        if (r < valid) {
            bf16x8 out;
#pragma unroll
            for (int j = 0; j < 8; ++j) out[j] = (bf16)(x[j] * inv * sigmoidf_((float)gk[p][j]));
            *reinterpret_cast<bf16x8*>(yb + (unsigned)r * rs + 16u * (unsigned)(l & 15)) = out;
        }
    }
}

// Second part: S <- Diag(e^{G_C}) S + K~^T V_new.
template <int NTW, class L>
__device__ __forceinline__ void chain_b(f32x4 (&xs)[8][NTW], const bf16x8 (&yb)[2][NTW], const bf16* KGT,
                                        const float* egc) {
    typedef Mfma<bf16> MF;
    const int g = lane_id() >> 4;
    // fragments read two row tiles ahead: one tile's four MFMAs do not
    // cover an LDS read under load
    MF::frag kf[3][2];
    f32x4 dv[3];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        kf[p][0] = load_frag<bf16>(KGT, L::LC, p * 16, 0);
        kf[p][1] = load_frag<bf16>(KGT, L::LC, p * 16, 32);
        dv[p] = *reinterpret_cast<const f32x4*>(egc + p * 16 + 4 * g);
    }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
        const int cur = rt % 3, nxt = (rt + 2) % 3;
        if (rt + 2 < 8) {
            kf[nxt][0] = load_frag<bf16>(KGT, L::LC, (rt + 2) * 16, 0);
            kf[nxt][1] = load_frag<bf16>(KGT, L::LC, (rt + 2) * 16, 32);
            dv[nxt] = *reinterpret_cast<const f32x4*>(egc + (rt + 2) * 16 + 4 * g);
        }
#pragma unroll
        for (int ct = 0; ct < NTW; ++ct) {
            xs[rt][ct] *= dv[cur];
            xs[rt][ct] = MF::mma(kf[cur][0], yb[0][ct], xs[rt][ct]);
            xs[rt][ct] = MF::mma(kf[cur][1], yb[1][ct], xs[rt][ct]);
        }
    }
}

// One chunk's tokens as a gate wave loads them: rows 16R + i, channels 2l,
// 2l+1 (v likewise); beta of row l.
template <bool HASQ>
struct PIn {
    bf16x2 z[SUB], k[SUB], q[HASQ ? SUB : 1];
    bf16 beta;
};
// v of rows 16R + i, channels 2l, 2l+1, as the wave that writes v^T loads it:
// the state waves for EXPAND (fewer live registers in the gate waves, which
// hold q), the gate waves for COMPOSE (whose state waves hold P and R).
struct PV {
    bf16x2 v[SUB];
};

// The scalar gate (SG, one logit per token and head, z of shape (B, T, H)):
// lane l holds the logit of row 16R + l%16 (in both halves of z[0]).
__device__ __forceinline__ bf16x2 pfetch_zs(const bf16* __restrict__ z, size_t row0, int valid, int H, int R) {
    const bf16 x = z[row0 + (size_t)min(SUB * R + (lane_id() & 15), valid - 1) * H];
    return bf16x2{x, x};
}

template <bool HASQ, bool SG = false>
__device__ __forceinline__ void pfetch_zkq(PIn<HASQ>& r, const bf16* __restrict__ q, const bf16* __restrict__ k,
                                           const bf16* __restrict__ z, const bf16* __restrict__ beta, size_t row0,
                                           int valid, int H, int R) {
    const int l = lane_id(), last = valid - 1;
    if constexpr (SG) r.z[0] = pfetch_zs(z, row0, valid, H, R);
    // wave-uniform chunk bases and 32-bit byte offsets (row, clamped to the
    // last token, then the lane's two channels): scalar-base addressing
    const char* zb = reinterpret_cast<const char*>(z + row0 * 128);
    const char* kb = reinterpret_cast<const char*>(k + row0 * 128);
    const char* qb = reinterpret_cast<const char*>(q + row0 * 128);
    const unsigned lo = 4u * (unsigned)l, rstride = (unsigned)H * 256u;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const unsigned off = (unsigned)min(SUB * R + i, last) * rstride + lo;
        if constexpr (!SG) r.z[i] = *reinterpret_cast<const bf16x2*>(zb + off);
        r.k[i] = *reinterpret_cast<const bf16x2*>(kb + off);
        if constexpr (HASQ) r.q[i] = *reinterpret_cast<const bf16x2*>(qb + off);
    }
    r.beta = beta[row0 + (size_t)min(l, last) * H];
}

// The same loads in two parts: z alone, then k, q and beta.
template <bool HASQ, bool SG = false>
__device__ __forceinline__ void pfetch_z(PIn<HASQ>& r, const bf16* __restrict__ z, size_t row0, int valid, int H,
                                         int R) {
    if constexpr (SG) {
        r.z[0] = pfetch_zs(z, row0, valid, H, R);
        return;
    }
    const int last = valid - 1;
    const char* zb = reinterpret_cast<const char*>(z + row0 * 128);
    const unsigned lo = 4u * (unsigned)lane_id(), rstride = (unsigned)H * 256u;
#pragma unroll
    for (int i = 0; i < SUB; ++i)
        r.z[i] = *reinterpret_cast<const bf16x2*>(zb + (unsigned)min(SUB * R + i, last) * rstride + lo);
}

template <bool HASQ>
__device__ __forceinline__ void pfetch_kq(PIn<HASQ>& r, const bf16* __restrict__ q, const bf16* __restrict__ k,
                                          const bf16* __restrict__ beta, size_t row0, int valid, int H, int R) {
    const int l = lane_id(), last = valid - 1;
    const char* kb = reinterpret_cast<const char*>(k + row0 * 128);
    const char* qb = reinterpret_cast<const char*>(q + row0 * 128);
    const unsigned lo = 4u * (unsigned)l, rstride = (unsigned)H * 256u;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const unsigned off = (unsigned)min(SUB * R + i, last) * rstride + lo;
        r.k[i] = *reinterpret_cast<const bf16x2*>(kb + off);
        if constexpr (HASQ) r.q[i] = *reinterpret_cast<const bf16x2*>(qb + off);
    }
    r.beta = beta[row0 + (size_t)min(l, last) * H];
}

// Rows at or past `valid` of a ragged last chunk become identity tokens:
// z = -inf (a zero gate, alpha = 1) and k = q = 0 (no write, no read); beta
// is set to 0 where it is stored.
template <bool HASQ, bool SG = false>
__device__ __forceinline__ void pmask(PIn<HASQ>& r, int valid, int R) {
    if constexpr (SG) {   // the lane's own row
        const unsigned keep = SUB * R + (lane_id() & 15) < valid ? 0xffffffffu : 0u;
        r.z[0] = __builtin_bit_cast(bf16x2, (__builtin_bit_cast(unsigned, r.z[0]) & keep) | (0xff80ff80u & ~keep));
    }
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const unsigned keep = SUB * R + i < valid ? 0xffffffffu : 0u;
        if constexpr (!SG)
            r.z[i] = __builtin_bit_cast(bf16x2, (__builtin_bit_cast(unsigned, r.z[i]) & keep) | (0xff80ff80u & ~keep));
        r.k[i] = __builtin_bit_cast(bf16x2, __builtin_bit_cast(unsigned, r.k[i]) & keep);
        if constexpr (HASQ) r.q[i] = __builtin_bit_cast(bf16x2, __builtin_bit_cast(unsigned, r.q[i]) & keep);
    }
}

__device__ __forceinline__ void pfetch_v(PV& r, const bf16* __restrict__ v, size_t row0, int valid, int H, int R) {
    const int last = valid - 1;
    const char* vb = reinterpret_cast<const char*>(v + row0 * 128);
    const unsigned lo = 4u * (unsigned)lane_id(), rstride = (unsigned)H * 256u;
#pragma unroll
    for (int i = 0; i < SUB; ++i)
        r.v[i] = *reinterpret_cast<const bf16x2*>(vb + (unsigned)min(SUB * R + i, last) * rstride + lo);
}

// S[i] = running sum of sigmoid(z) over the block's rows (registers only);
// the log2 decay is G = kg2 S.
// With the scalar gate the block's 16 rows are spread over the lanes of each
// DPP row (lane l: row l%16): sigmoid once per lane, then the running sum
// passed down the lanes one at a time, so that every partial sum is formed
// in the same order, with the same roundings, as the per-channel loop below;
// `own` keeps the lane's own row's sum, S[i] every row's (wave-uniform).
template <bool HASQ, bool SG = false>
__device__ __forceinline__ void gate_sums(const PIn<HASQ>& in, float (&S)[SUB][2], float& own) {
    if constexpr (SG) {
        const int lr = lane_id() & 15;
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * (float)in.z[0][0]));
        float x = 0.f + sg;
#pragma unroll
        for (int t = 1; t < SUB; ++t) {   // row_shr:1 -- lane t takes lane t-1's finished sum
            const float prev =
                __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, false));
            x = lr == t ? prev + sg : x;
        }
        own = x;
#pragma unroll
        for (int i = 0; i < SUB; ++i)
            S[i][0] = S[i][1] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), i));
        return;
    }
    (void)own;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        s0 += __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * (float)in.z[i][0]));
        s1 += __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * (float)in.z[i][1]));
        S[i][0] = s0;
        S[i][1] = s1;
    }
}

// The rest of S1: block sums and references, beta, the block-local factors
// e^{+-(G_r - G_m(R))} and the operands k e^{G-G_m} (not needed without the
// solve), k e^{G_m-G}, q e^{G-G_m}.
template <int MODE, bool SG = false>
__device__ __forceinline__ void gate_rest(const PIn<MODE != COMPOSE>& in, int R, int valid, float kg2,
                                          unsigned char* smem, const float (&S)[SUB][2], float own,
                                          float (&kl)[SUB][2], float (&kr)[SUB][2],
                                          float (&ql)[MODE != COMPOSE ? SUB : 1][2]) {
    typedef PLay<MODE> L;
    constexpr bool EXP = L::EXP;
    constexpr int LDK = L::LDK;
    const int l = lane_id(), c0 = 2 * l;
    bf16* KL = reinterpret_cast<bf16*>(smem + L::OFF_KL);
    bf16* KR = reinterpret_cast<bf16*>(smem + L::OFF_KR);
    bf16* QL = reinterpret_cast<bf16*>(smem + L::OFF_QL);
    float* tot = reinterpret_cast<float*>(smem + L::OFF_TOT);
    float* mloc = reinterpret_cast<float*>(smem + L::OFF_MLOC);
    float* bet = reinterpret_cast<float*>(smem + L::OFF_BET);
    const float m0 = kg2 * S[7][0], m1 = kg2 * S[7][1];
    *reinterpret_cast<float2*>(tot + R * 128 + c0) = float2{kg2 * S[SUB - 1][0], kg2 * S[SUB - 1][1]};
    *reinterpret_cast<float2*>(mloc + R * 128 + c0) = float2{m0, m1};
    if ((l >> 4) == R) bet[l] = l < valid ? (float)in.beta : 0.f;
    // scalar gate: each lane forms its own row's factors, which every lane
    // then reads (wave-uniform)
    float lf = 0.f, rf = 0.f;
    if constexpr (SG) {
        const float el = __builtin_fmaf(kg2, own, -m0);
        lf = __builtin_amdgcn_exp2f(el);
        rf = __builtin_amdgcn_exp2f(-el);
    }
    (void)own;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const int r = SUB * R + i;
        float lsg = 0.f, rsg = 0.f;
        if constexpr (SG) {
            lsg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lf), i));
            rsg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rf), i));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float left, right;
            if constexpr (SG) {
                left = lsg;
                right = rsg;
            } else {
                const float el = __builtin_fmaf(kg2, S[i][j], -(j ? m1 : m0));   // G_r - G_m(R)
                left = __builtin_amdgcn_exp2f(el);
                right = __builtin_amdgcn_exp2f(-el);
            }
            const float kv = (float)in.k[i][j];
            kl[i][j] = kv * left;
            kr[i][j] = kv * right;
            if constexpr (EXP) ql[i][j] = (float)in.q[i][j] * left;
        }
        if constexpr (L::SOLVE) store2<bf16>(KL + r * LDK + c0, kl[i][0], kl[i][1]);
        store2<bf16>(KR + r * LDK + c0, kr[i][0], kr[i][1]);
        if constexpr (EXP) store2<bf16>(QL + r * LDK + c0, ql[i][0], ql[i][1]);
    }
}

// S1 of gate wave R (rows past the end have been made identity tokens).  On
// return kl, kr, ql hold the block's decay-scaled k and q (fp32).
template <int MODE, bool SG = false>
__device__ __forceinline__ void pipe_gate(const PIn<MODE != COMPOSE>& in, int R, int valid, float kg2,
                                          unsigned char* smem, float (&kl)[SUB][2], float (&kr)[SUB][2],
                                          float (&ql)[MODE != COMPOSE ? SUB : 1][2]) {
    float S[SUB][2], own;
    gate_sums<MODE != COMPOSE, SG>(in, S, own);
    gate_rest<MODE, SG>(in, R, valid, kg2, smem, S, own, kl, kr, ql);
}

// S2 of gate wave R: A_RR (and M_RR) from the block's own rows of KL, KR,
// QL, transposed: lane holds row r = 16R + l%16, key indices 16R + 4(l/16) + e.
// Issued first, so that pipe_abs runs while the products are in flight.
template <int MODE>
__device__ __forceinline__ void pipe_diag_mma(int R, const unsigned char* smem, f32x4& accA, f32x4& accM) {
    typedef PLay<MODE> L;
    typedef Mfma<bf16> MF;
    constexpr int LDK = L::LDK;
    const bf16* KL = reinterpret_cast<const bf16*>(smem + L::OFF_KL);
    const bf16* KR = reinterpret_cast<const bf16*>(smem + L::OFF_KR);
    const bf16* QL = reinterpret_cast<const bf16*>(smem + L::OFF_QL);
    accA = zero4();
    accM = zero4();
#pragma unroll
    for (int kk = 0; kk < 128; kk += MF::KSTEP) {
        const MF::frag ak = load_frag<bf16>(KR, LDK, R * SUB, kk);
        if constexpr (L::SOLVE) accA = MF::mma(ak, load_frag<bf16>(KL, LDK, R * SUB, kk), accA);
        if constexpr (L::EXP) accM = MF::mma(ak, load_frag<bf16>(QL, LDK, R * SUB, kk), accM);
    }
}

// Then beta_r A~_RR (strictly lower) and M_RR into LDS, and
// D'_R = (I + beta_R A~_RR)^{-1} diag(beta_R).
template <int MODE>
__device__ __forceinline__ void pipe_diag_inv(int R, unsigned char* smem, const f32x4& accA, f32x4 accM) {
    typedef PLay<MODE> L;
    constexpr int LT = L::LT, LB = L::LB, BS = L::BS;
    int l = lane_id();
    asm volatile("" : "+v"(l));   // keep lane-derived constants out of the loop preheader
    bf16* Ms = reinterpret_cast<bf16*>(smem + L::OFF_M);
    float* As = reinterpret_cast<float*>(smem + L::OFF_AS);
    bf16* Db = reinterpret_cast<bf16*>(smem + L::OFF_DB);
    const float* bet = reinterpret_cast<const float*>(smem + L::OFF_BET);
    const int rr = l & 15, ii = 4 * (l >> 4);
    if constexpr (L::EXP) {
#pragma unroll
        for (int e = 0; e < 4; ++e) accM[e] = (ii + e <= rr) ? accM[e] : 0.f;
        store4p(Ms + (R * SUB + rr) * LT + pcol(R * SUB + ii), accM[0], accM[1], accM[2], accM[3]);
    }
    if constexpr (L::SOLVE) {
        const float br = bet[R * SUB + rr];
#pragma unroll
        for (int e = 0; e < 4; ++e) As[R * BS + (ii + e) * SUB + rr] = (ii + e < rr) ? br * accA[e] : 0.f;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // this wave's As stores

        // lane = column, right-looking substitution down the column (lanes
        // 16.. repeat lanes 0..15)
        const int col = l & 15;
        const float* at = As + R * BS;   // at[i * 16 + r] = beta_r A~_ri
        float x[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) x[r] = (r == col) ? 1.f : 0.f;
        inv_batch<0, 3>(at, x);
        inv_batch<3, 7>(at, x);
        inv_batch<7, 11>(at, x);
        inv_batch<11, 15>(at, x);
        if (l < 16) {
            const float bc = bet[R * SUB + col];
            bf16* d = Db + R * SUB * LB + col;
#pragma unroll
            for (int r = 0; r < SUB; ++r) d[r * LB] = (bf16)(x[r] * bc);
        }
    }
}

// S2 of gate wave R: absolute block references from the block sums, then the
// chain operands of block R.
// v^T of rows 16R..16R+15 as loaded (rows past the end meet beta = 0 in the solve).
template <int MODE>
__device__ __forceinline__ void pipe_vt(const PV& pv, int R, unsigned char* smem) {
    typedef PLay<MODE> L;
    constexpr int LC = L::LC;
    const int c0 = 2 * lane_id();
    bf16* RV = reinterpret_cast<bf16*>(smem + L::OFF_RV);
#pragma unroll
    for (int i = 0; i < SUB; i += 4)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *reinterpret_cast<bf16x4*>(RV + (c0 + j) * LC + SUB * R + i) =
                bf16x4{pv.v[i][j], pv.v[i + 1][j], pv.v[i + 2][j], pv.v[i + 3][j]};
}

template <int MODE>
__device__ __forceinline__ void pipe_abs(int R, unsigned char* smem,
                                         const float (&kl)[SUB][2], const float (&kr)[SUB][2],
                                         const float (&ql)[MODE != COMPOSE ? SUB : 1][2], int buf) {
    typedef PLay<MODE> L;
    constexpr bool EXP = L::EXP;
    constexpr int LDK = L::LDK, LC = L::LC;
    const int l = lane_id(), c0 = 2 * l;
    bf16* KGn = reinterpret_cast<bf16*>(smem + L::OFF_KG);
    bf16* QG = reinterpret_cast<bf16*>(smem + L::OFF_QG);
    bf16* KGT = reinterpret_cast<bf16*>(smem + L::OFF_KGT + buf * L::KGT_SZ);
    float* egc = reinterpret_cast<float*>(smem + L::OFF_EGC + buf * 128 * 4);
    const float* tot = reinterpret_cast<const float*>(smem + L::OFF_TOT);
    const float* mloc = reinterpret_cast<const float*>(smem + L::OFF_MLOC);

    float gR[2] = {0.f, 0.f}, gC[2] = {0.f, 0.f};   // G before block R; G_C
#pragma unroll
    for (int B = 0; B < 4; ++B) {
        const float2 t = *reinterpret_cast<const float2*>(tot + B * 128 + c0);
        if (B < R) {
            gR[0] += t.x;
            gR[1] += t.y;
        }
        gC[0] += t.x;
        gC[1] += t.y;
    }
    const float2 ml = *reinterpret_cast<const float2*>(mloc + R * 128 + c0);
    const float mR[2] = {gR[0] + ml.x, gR[1] + ml.y};
    float eGm[2], eCGm[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        eGm[j] = __builtin_amdgcn_exp2f(mR[j]);
        eCGm[j] = __builtin_amdgcn_exp2f(gC[j] - mR[j]);
    }
    if (R == 0) *reinterpret_cast<float2*>(egc + c0) = float2{__builtin_amdgcn_exp2f(gC[0]),
                                                              __builtin_amdgcn_exp2f(gC[1])};
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const int r = SUB * R + i;
        store2<bf16>(KGn + r * LDK + pcol(c0), -kl[i][0] * eGm[0], -kl[i][1] * eGm[1]);
        if constexpr (EXP) store2<bf16>(QG + r * LDK + pcol(c0), ql[i][0] * eGm[0], ql[i][1] * eGm[1]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < SUB; i += 4)
            store4p(KGT + (c0 + j) * LC + pcol(SUB * R + i), kr[i][j] * eCGm[j], kr[i + 1][j] * eCGm[j],
                    kr[i + 2][j] * eCGm[j], kr[i + 3][j] * eCGm[j]);
}

// Off-diagonal block pairs (R, I), I < R, per state wave: two each for waves
// 0-1, one each for waves 2-3.
__constant__ int kPipePairs[4][2][2] = {{{1, 0}, {3, 0}}, {{2, 0}, {3, 1}}, {{2, 1}, {-1, -1}}, {{3, 2}, {-1, -1}}};

// S2 of a state wave: the cross-block factors e^{(G_m(R) - G_m(I)) / 2} of its NP
// pairs into LDS (read back by the same wave only), then -A~_RI (without the
// row factor beta_r, which the inverses carry) and M_RI, the NP pairs
// interleaved in one pass over the key channels.
template <int MODE, int NP>
__device__ __forceinline__ void pipe_pairs(int w, unsigned char* smem) {
    typedef PLay<MODE> L;
    typedef Mfma<bf16> MF;
    constexpr int LDK = L::LDK, LT = L::LT, LB = L::LB, DK = L::DK;
    int l = lane_id();
    asm volatile("" : "+v"(l));   // keep lane-derived constants out of the loop preheader
    const bf16* KL = reinterpret_cast<const bf16*>(smem + L::OFF_KL);
    const bf16* KR = reinterpret_cast<const bf16*>(smem + L::OFF_KR);
    const bf16* QL = reinterpret_cast<const bf16*>(smem + L::OFF_QL);
    bf16* Ms = reinterpret_cast<bf16*>(smem + L::OFF_M);
    bf16* Ab = reinterpret_cast<bf16*>(smem + L::OFF_AB);
    float* dsc = reinterpret_cast<float*>(smem + L::OFF_DSC);
    const float* tot = reinterpret_cast<const float*>(smem + L::OFF_TOT);
    const float* mloc = reinterpret_cast<const float*>(smem + L::OFF_MLOC);
    const int c0 = 2 * l;
    int Rp[NP], Ip[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        Rp[j] = kPipePairs[w][j][0];
        Ip[j] = kPipePairs[w][j][1];
        const int R = Rp[j], I = Ip[j];
        // G_m(R) - G_m(I) = (block sums I..R-1) + mloc_R - mloc_I
        const float2 mr = *reinterpret_cast<const float2*>(mloc + R * 128 + c0);
        const float2 mi = *reinterpret_cast<const float2*>(mloc + I * 128 + c0);
        float d0 = mr.x - mi.x, d1 = mr.y - mi.y;
#pragma unroll
        for (int B = 0; B < 3; ++B)
            if (B >= I && B < R) {
                const float2 t = *reinterpret_cast<const float2*>(tot + B * 128 + c0);
                d0 += t.x;
                d1 += t.y;
            }
        *reinterpret_cast<float2*>(dsc + (R * (R - 1) / 2 + I) * DK + c0) =
            float2{__builtin_amdgcn_exp2f(0.5f * d0), __builtin_amdgcn_exp2f(0.5f * d1)};   // applied twice
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // this wave's dsc rows
    f32x4 accA[NP], accM[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) accA[j] = accM[j] = zero4();
#pragma unroll
    for (int kk = 0; kk < DK; kk += MF::KSTEP) {
        const int cc = kk + (l >> 4) * MF::KPL;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int R = Rp[j], I = Ip[j];
            const float* dv = dsc + (R * (R - 1) / 2 + I) * DK + cc;
            MF::frag ak = load_frag<bf16>(KR, LDK, I * SUB, kk);
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(dv), d1 = *reinterpret_cast<const f32x4*>(dv + 4);
            float t[MF::KPL];
            MF::to_floats(ak, t);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                t[jj] = (t[jj] * d0[jj]) * d0[jj];
                t[jj + 4] = (t[jj + 4] * d1[jj]) * d1[jj];
            }
            ak = MF::from_floats(t);
            if constexpr (L::SOLVE) accA[j] = MF::mma(ak, load_frag<bf16>(KL, LDK, R * SUB, kk), accA[j]);
            if constexpr (L::EXP) accM[j] = MF::mma(ak, load_frag<bf16>(QL, LDK, R * SUB, kk), accM[j]);
        }
    }
    const int rr = l & 15, ii = 4 * (l >> 4);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int R = Rp[j], I = Ip[j];
        if constexpr (L::SOLVE)
            store4p(Ab + ((R * (R - 1) / 2 + I) * SUB + rr) * LB + ii, -accA[j][0], -accA[j][1], -accA[j][2],
                    -accA[j][3]);
        if constexpr (L::EXP)
            store4p(Ms + (R * SUB + rr) * LT + pcol(I * SUB + ii), accM[j][0], accM[j][1], accM[j][2], accM[j][3]);
    }
}

// S3: column block wT of T' = (I + A)^{-1} diag(beta) by block forward
// substitution on the identity's columns: X_R = D'_R (E_R - sum_{J<R} A~_RJ X_J).
template <int MODE>
__device__ __forceinline__ void pipe_tsolve(int wT, unsigned char* smem) {
    typedef PLay<MODE> L;
    constexpr int LT = L::LT, LB = L::LB;
    int l = lane_id();
    asm volatile("" : "+v"(l));
    const int g = l >> 4, c = l & 15;
    const bf16* Ab = reinterpret_cast<const bf16*>(smem + L::OFF_AB);
    const bf16* Db = reinterpret_cast<const bf16*>(smem + L::OFF_DB);
    bf16* Tp = reinterpret_cast<bf16*>(smem + L::OFF_TP);
    bf16x4 ab[6], db[4];
#pragma unroll
    for (int p = 0; p < 6; ++p) ab[p] = *reinterpret_cast<const bf16x4*>(Ab + (p * SUB + c) * LB + 4 * g);
#pragma unroll
    for (int R = 0; R < 4; ++R) db[R] = *reinterpret_cast<const bf16x4*>(Db + (R * SUB + c) * LB + 4 * g);
    f32x4 eye;
#pragma unroll
    for (int e = 0; e < 4; ++e) eye[e] = (4 * g + e == c) ? 1.f : 0.f;
    bf16x4 xb[4];
    bf16* tcol = Tp + 4 * g * LT + pcol(16 * wT + c);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        f32x4 x = zero4();
        if (R >= wT) {
            f32x4 acc = (R == wT) ? eye : zero4();
#pragma unroll
            for (int J = 0; J < R; ++J)
                if (J >= wT) acc = mma16(ab[R * (R - 1) / 2 + J], xb[J], acc);
            x = mma16(db[R], to_bf4(acc), zero4());
        }
        xb[R] = to_bf4(x);
#pragma unroll
        for (int e = 0; e < 4; ++e) tcol[(R * SUB + e) * LT] = xb[R][e];
    }
}

// Same grid and arguments as seg_kernel, plus tm: the per-chunk T'
// ([chain][chunk] x TM_ELEMS bf16) that COMPOSE writes and EXPAND_LITE reads
// (unused by EXPAND, which forms it itself).  GATED (EXPAND_LITE): the
// output epilogue y = RMSNorm(o) * sigmoid(gate) is fused, with gate and y
// laid out like o; o is written only when not NULL.  Chunk m's outputs are
// staged in LDS in S1 and its epilogue runs in S2, on the state waves (rows
// 0-15 on waves 0-1, whose M pairs are the longer, rows 16-63 on waves 2-3).
// SG: the scalar gate (z holds one logit per token and head, shape (B, T, H)).
// The body of one workgroup: segment `seg` of chain `bh`.
template <int MODE, bool GATED = false, bool SG = false>
__device__ __forceinline__ void pipe_run(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                         const bf16* __restrict__ v, const bf16* __restrict__ z,
                                         const bf16* __restrict__ beta, float g_min, int T, int H, int NC, int L,
                                         int nchain, const float* __restrict__ xin, float* __restrict__ xo0,
                                         float* __restrict__ xo1, bf16* __restrict__ o, bf16* __restrict__ tm,
                                         const bf16* __restrict__ gate, float eps, bf16* __restrict__ y, const int seg,
                                         const size_t bh) {
    static_assert(!GATED || MODE == EXPAND_LITE, "the epilogue is fused into the light expand only");
    typedef PLay<MODE> LY;
    constexpr int DK = 128, DV = 128;
    constexpr bool EXP = LY::EXP, LITE = LY::LITE;
    // v^T is written by the state waves in EXPAND, by the gate waves otherwise
    constexpr bool VSTATE = MODE == EXPAND;
    extern __shared__ __align__(16) unsigned char smem[];
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int l = lane_id(), w = wave_id();
    __builtin_assume(w >= 0 && w < NTH / 64);
    const int n0 = seg * L, n1 = min(NC, n0 + L), nL = n1 - n0;
    auto row_of = [&](int n) __attribute__((always_inline)) { return ((size_t)b * T + (size_t)n * C) * H + h; };
    auto tm_of = [&](int n) __attribute__((always_inline)) { return tm + (bh * NC + n) * TM_ELEMS; };

    if constexpr (EXP) {
        // strictly upper blocks of M stay zero
        if (w >= 2) {
            const int p = w - 2;
            const int R = p < 3 ? 0 : (p < 5 ? 1 : 2);
            const int I = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
            store4p(reinterpret_cast<bf16*>(smem + LY::OFF_M) + (R * SUB + (l & 15)) * LY::LT +
                        pcol(I * SUB + 4 * (l >> 4)),
                    0.f, 0.f, 0.f, 0.f);
        }
    }

    if (w < 4) {
        // ---------------- state waves
        constexpr int NH = EXP ? 1 : 2;          // 32-column halves per wave
        const bool ptile = !EXP && w < 2;
        const bool hasu = EXP || !ptile;
        const int NX = ptile ? DK : DV;
        const int cbase = EXP ? 32 * w : 64 * (w & 1);
        const size_t xblk = ((size_t)seg * nchain + bh) * DK;
        f32x4 xs[NH][DK / 16][2];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = rt * 16 + 4 * (l >> 4) + e, col = cbase + 32 * hh + ct * 16 + (l & 15);
                        float x = 0.f;
                        if constexpr (EXP) x = xin ? xin[(xblk + row) * DV + col] : 0.f;
                        else x = (ptile && row == col) ? 1.f : 0.f;
                        xs[hh][rt][ct][e] = x;
                    }
        const size_t ostride = (size_t)H * DV;
        PV pv;
        if constexpr (VSTATE) pfetch_v(pv, v, row_of(n0), min(C, T - n0 * C), H, w);
        bf16x8 yb[NH][2][2];
        // GATED: chunk n's gate logits for this wave's rows, then its y
        bf16x8 gk[6];
        const int er0 = w < 2 ? 8 * w : 16 + 24 * (w - 2);
        auto fetch_gate = [&](int n) __attribute__((always_inline)) {
            const bf16* g0 = gate + row_of(n) * DV;
            if (w < 2)
                gate_fetch<2>(gk, g0, er0, min(C, T - n * C), ostride);
            else
                gate_fetch<6>(gk, g0, er0, min(C, T - n * C), ostride);
        };
        auto epilogue = [&](int n) __attribute__((always_inline)) {
            bf16* y0 = y + row_of(n) * DV;
            if (w < 2)
                gate_epilogue<2, LY>(gk, smem, eps, y0, er0, min(C, T - n * C), ostride);
            else
                gate_epilogue<6, LY>(gk, smem, eps, y0, er0, min(C, T - n * C), ostride);
        };
        // state update of chunk n from V_new in yb (COMPOSE defers it to S3)
        auto update = [&](int n) __attribute__((always_inline)) {
            const int bufn = LY::NKB == 2 ? (n & 1) : 0;
            const bf16* KGT = reinterpret_cast<const bf16*>(smem + LY::OFF_KGT + bufn * LY::KGT_SZ);
            const float* egc = reinterpret_cast<const float*>(smem + LY::OFF_EGC + bufn * 128 * 4);
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                chain_b<2, LY>(xs[hh], yb[hh], KGT, egc);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto chain = [&](int m) __attribute__((always_inline)) {
            // COMPOSE hands the chunk's T' (complete since the last barrier)
            // to the expand pass
            if constexpr (MODE == COMPOSE) {
                f32x4* g = reinterpret_cast<f32x4*>(tm_of(m));
#pragma unroll
                for (int j = 0; j < 2; ++j) g[threadIdx.x + 256 * j] = *tp_lds<LY>(smem, threadIdx.x + 256 * j);
            }
            const int valid = min(C, T - m * C);
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                const int col0 = cbase + 32 * hh;
                chain_a<MODE, 2, LY, GATED>(xs[hh], yb[hh], hasu, col0, smem, o ? o + row_of(m) * DV + col0 : nullptr,
                                            valid, ostride);
                __builtin_amdgcn_sched_barrier(0);   // one half's working set at a time
            }
        };
        // the state waves' share of the steps after S1 for chunk n
        // (COMPOSE: the previous chunk's state update in S3, while the gate
        // waves solve for T')
        auto rest = [&](int n, bool upd) __attribute__((always_inline)) {
            // EXPAND_LITE: chunk n's T' from the compose pass, into LDS after
            // the M pairs (the state waves have room in S2; the gate waves'
            // S1 is the longer step)
            f32x4 tpr[LITE ? 2 : 1];
            if constexpr (LITE) {
                const f32x4* tg = reinterpret_cast<const f32x4*>(tm_of(n));
#pragma unroll
                for (int j = 0; j < 2; ++j) tpr[j] = tg[threadIdx.x + 256 * j];
            }
            if constexpr (GATED)
                if (upd) fetch_gate(n - 1);
            if constexpr (VSTATE) {
                pipe_vt<MODE>(pv, w, smem);
                const int mn = min(n + 1, n1 - 1);
                pfetch_v(pv, v, row_of(mn), min(C, T - mn * C), H, w);
            }
            if (w < 2)
                pipe_pairs<MODE, 2>(w, smem);
            else
                pipe_pairs<MODE, 1>(w, smem);
            if constexpr (LITE) {
#pragma unroll
                for (int j = 0; j < 2; ++j) *tp_lds<LY>(smem, threadIdx.x + 256 * j) = tpr[j];
            }
            if constexpr (GATED)
                if (upd) epilogue(n - 1);
            if constexpr (!LITE) {
                __syncthreads();   // S2 | S3
                if constexpr (!EXP) {
                    if (upd) update(n - 1);
                } else {
                    pipe_tsolve<MODE>(w, smem);   // the gate waves form the next chunk's sums meanwhile
                }
            }
            __syncthreads();   // S3 (S2 for EXPAND_LITE) | next S1
        };
        // iteration 0 has no step to run; iterations 1.. run the step of the
        // previous chunk in S1 (COMPOSE: its state update in S3)
        __syncthreads();   // S1 | S2
        rest(n0, false);
        for (int i = 1; i < nL; ++i) {
            const int m = n0 + i;
            chain(m - 1);
            if constexpr (EXP) update(m - 1);
            __syncthreads();   // S1 | S2
            rest(m, true);
        }
        chain(n1 - 1);
        if constexpr (GATED) fetch_gate(n1 - 1);
        update(n1 - 1);
        if constexpr (GATED) {
            __syncthreads();   // every wave's sums of squares of the last chunk
            epilogue(n1 - 1);
        }
        float* xo = EXP ? xo0 : (ptile ? xo0 : xo1);
        if (xo) {
            const size_t ob = EXP ? bh * DK : xblk;
#pragma unroll
            for (int hh = 0; hh < NH; ++hh)
#pragma unroll
                for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = rt * 16 + 4 * (l >> 4) + e;
                            const int col = cbase + 32 * hh + ct * 16 + (l & 15);
                            xo[(ob + row) * NX + col] = xs[hh][rt][ct][e];
                        }
        }
    } else if constexpr (EXP) {
        // ---------------- gate waves, EXPAND and EXPAND_LITE: block R of each
        // chunk.  The next chunk's running sums of sigmoid(z) are formed in
        // the last step (S2 for EXPAND_LITE, where the state waves' M pairs
        // leave room; S3 for EXPAND, where the state waves solve for T') and
        // kept in registers.
        const int R = w - 4;
        const float kg2 = g_min * LOG2E;
        PIn<true> in;
        PV pv;
        float S[SUB][2], own;
        {
            const int valid = min(C, T - n0 * C);
            pfetch_zkq<true, SG>(in, q, k, z, beta, row_of(n0), valid, H, R);
            if constexpr (LITE) pfetch_v(pv, v, row_of(n0), valid, H, R);
            if (valid < C) pmask<true, SG>(in, valid, R);
            gate_sums<true, SG>(in, S, own);
        }
        float kl[SUB][2], kr[SUB][2], ql[SUB][2];
        for (int i = 0; i < nL; ++i) {
            const int m = n0 + i;
            const int valid = min(C, T - m * C);
            const int mn = min(m + 1, n1 - 1);   // prefetch target, clamped (unconditional)
            const int valid_n = min(C, T - mn * C);
            pfetch_z<true, SG>(in, z, row_of(mn), valid_n, H, R);   // this chunk's z is consumed
            gate_rest<MODE, SG>(in, R, valid, kg2, smem, S, own, kl, kr, ql);
            pfetch_kq<true>(in, q, k, beta, row_of(mn), valid_n, H, R);
            __syncthreads();   // S1 | S2
            f32x4 accA, accM;
            pipe_diag_mma<MODE>(R, smem, accA, accM);
            pipe_abs<MODE>(R, smem, kl, kr, ql, 0);
            if constexpr (LITE) pipe_vt<MODE>(pv, R, smem);
            pipe_diag_inv<MODE>(R, smem, accA, accM);
            if constexpr (LITE) {
                pfetch_v(pv, v, row_of(mn), valid_n, H, R);
            } else {
                __syncthreads();   // S2 | S3
            }
            if (valid_n < C) pmask<true, SG>(in, valid_n, R);
            gate_sums<true, SG>(in, S, own);
            __syncthreads();   // S2 (S3 for EXPAND) | next S1
        }
        if constexpr (GATED) __syncthreads();   // the state waves' last epilogue
    } else {
        // ---------------- gate waves, COMPOSE: block R of each chunk
        const int R = w - 4;
        const float kg2 = g_min * LOG2E;
        PIn<false> in;
        PV pv;
        {
            const int valid = min(C, T - n0 * C);
            pfetch_zkq<false, SG>(in, q, k, z, beta, row_of(n0), valid, H, R);
            pfetch_v(pv, v, row_of(n0), valid, H, R);
        }
        float kl[SUB][2], kr[SUB][2], ql[1][2];
        for (int i = 0; i < nL; ++i) {
            const int m = n0 + i;
            const int valid = min(C, T - m * C);
            const int mn = min(m + 1, n1 - 1);   // prefetch target, clamped (unconditional)
            const int valid_n = min(C, T - mn * C);
            if (valid < C) pmask<false, SG>(in, valid, R);
            pipe_gate<MODE, SG>(in, R, valid, kg2, smem, kl, kr, ql);
            pfetch_zkq<false, SG>(in, q, k, z, beta, row_of(mn), valid_n, H, R);
            __syncthreads();   // S1 | S2
            f32x4 accA, accM;
            pipe_abs<MODE>(R, smem, kl, kr, ql, m & 1);
            pipe_diag_mma<MODE>(R, smem, accA, accM);
            pipe_diag_inv<MODE>(R, smem, accA, accM);
            __syncthreads();   // S2 | S3
            // v^T and the next chunk's v in S3, beside the state waves'
            // deferred update (S2 is the gate waves' longer step)
            pipe_vt<MODE>(pv, R, smem);
            pfetch_v(pv, v, row_of(mn), valid_n, H, R);
            pipe_tsolve<MODE>(R, smem);
            __syncthreads();   // S3 | next S1
        }
    }
}

template <int MODE, bool GATED = false, bool SG = false>
__global__ __launch_bounds__(NTH) void pipe_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                   const bf16* __restrict__ v, const bf16* __restrict__ z,
                                                   const bf16* __restrict__ beta, float g_min, int T, int H, int NC,
                                                   int L, int nchain, const float* __restrict__ xin,
                                                   float* __restrict__ xo0, float* __restrict__ xo1,
                                                   bf16* __restrict__ o, bf16* __restrict__ tm,
                                                   const bf16* __restrict__ gate, float eps, bf16* __restrict__ y) {
    pipe_run<MODE, GATED, SG>(q, k, v, z, beta, g_min, T, H, NC, L, nchain, xin, xo0, xo1, o, tm, gate, eps, y,
                              (int)(blockIdx.x / nchain), blockIdx.x % nchain);
}

// The split plan.  Segment 0 starts from s0, so it needs no transition: the
// first pass runs it as a full expand (outputs, and its end state as the
// entry state of segment 1) beside the compose of segments 1 .. nseg-2.  The
// last segment's transition is not needed either: the second pass runs it as
// a full expand from its entry state (outputs and s_final) beside the light
// expands of segments 1 .. nseg-2.  Segment `seg` of chain `bh` is workgroup
// (seg - first) * nchain + bh of its pass; P, R and the entry states E are
// indexed by segment as in the uniform plan (slots 0 and nseg-1 of P and R
// and slot 0 of E are not used).
template <bool SG>
__global__ __launch_bounds__(NTH) void pipe_first_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                         const bf16* __restrict__ v, const bf16* __restrict__ z,
                                                         const bf16* __restrict__ beta, float g_min, int T, int H,
                                                         int NC, int L, int nchain, const float* __restrict__ s0,
                                                         float* __restrict__ e1, float* __restrict__ P,
                                                         float* __restrict__ R, bf16* __restrict__ o,
                                                         bf16* __restrict__ tm) {
    const int seg = (int)(blockIdx.x / nchain);
    const size_t bh = blockIdx.x % nchain;
    if (seg == 0)
        pipe_run<EXPAND, false, SG>(q, k, v, z, beta, g_min, T, H, NC, L, nchain, s0, e1, nullptr, o, nullptr,
                                    nullptr, 0.f, nullptr, 0, bh);
    else
        pipe_run<COMPOSE, false, SG>(q, k, v, z, beta, g_min, T, H, NC, L, nchain, nullptr, P, R, nullptr, tm,
                                     nullptr, 0.f, nullptr, seg, bh);
}

// GATED: the light expands apply the output epilogue (y, and o when not
// NULL); the last segment's outputs go to o_end, for the epilogue kernel.
template <bool GATED, bool SG>
__global__ __launch_bounds__(NTH) void pipe_last_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                        const bf16* __restrict__ v, const bf16* __restrict__ z,
                                                        const bf16* __restrict__ beta, float g_min, int T, int H,
                                                        int NC, int L, int nchain, int nseg,
                                                        const float* __restrict__ E, float* __restrict__ s_final,
                                                        bf16* __restrict__ o, bf16* __restrict__ o_end,
                                                        bf16* __restrict__ tm, const bf16* __restrict__ gate,
                                                        float eps, bf16* __restrict__ y) {
    const int seg = (int)(blockIdx.x / nchain) + 1;
    const size_t bh = blockIdx.x % nchain;
    if (seg == nseg - 1)
        pipe_run<EXPAND, false, SG>(q, k, v, z, beta, g_min, T, H, NC, L, nchain, E, s_final, nullptr, o_end,
                                    nullptr, nullptr, 0.f, nullptr, seg, bh);
    else
        pipe_run<EXPAND_LITE, GATED, SG>(q, k, v, z, beta, g_min, T, H, NC, L, nchain, E, nullptr, nullptr, o, tm,
                                         gate, eps, y, seg, bh);
}

// ---------------------------------------------------------------------------
// Scan over segments for one chain and 16 state columns:
//   Sent[j] = S_j,  S_{j+1} = P_j S_j + R_j,  s_final = S_nseg.
// The products run on bf16 MFMA with both operands split into a high and a
// low bf16 part (x = hi + lo, |lo| <= 2^-9 |x|) and the three significant
// cross products accumulated in fp32, which keeps about 16 significant bits
// of P and S.  Wave w owns state rows 32w..32w+31; P_j's rows for the next
// segment are prefetched while the current one is applied.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = (bf16)a[i];
        hi[i + 4] = (bf16)b[i];
        lo[i] = (bf16)(a[i] - (float)hi[i]);
        lo[i + 4] = (bf16)(b[i] - (float)hi[i + 4]);
    }
}

template <int DK, int DV>
struct ScanIn {
    f32x4 p[2][DK / 32][2];   // P rows (32w + 16 rb + l%16), columns 32 kb + 8 (l/16) .. +7
    float r[2][4];            // R rows 32w + 16 rb + 4 (l/16) + e, column col0 + l%16
};

template <int DK, int DV>
__device__ __forceinline__ void scan_load(ScanIn<DK, DV>& in, const float* __restrict__ P, const float* __restrict__ R,
                                          int j, int nchain, size_t bh, int col0, int w, int l) {
    const size_t blk = ((size_t)j * nchain + bh) * DK;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float* prow = P + (blk + 32 * w + 16 * rb + (l & 15)) * DK + 8 * (l >> 4);
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            in.p[rb][kb][0] = *reinterpret_cast<const f32x4*>(prow + 32 * kb);
            in.p[rb][kb][1] = *reinterpret_cast<const f32x4*>(prow + 32 * kb + 4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            in.r[rb][e] = R[(blk + 32 * w + 16 * rb + 4 * (l >> 4) + e) * DV + col0 + (l & 15)];
    }
}

template <int DK, int DV>
__device__ __forceinline__ void scan_apply(f32x4 (&acc)[2], const ScanIn<DK, DV>& in, float* __restrict__ Sent,
                                           float* St, int j, int nchain, size_t bh, int col0, int w, int l) {
    constexpr int LS = DK + 4;
    typedef Mfma<bf16> MF;
    const size_t blk = ((size_t)j * nchain + bh) * DK;
    const int c = l & 15, g = l >> 4;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = 32 * w + 16 * rb + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) Sent[(blk + row + e) * DV + col0 + c] = acc[rb][e];
        *reinterpret_cast<f32x4*>(St + c * LS + row) = acc[rb];
    }
    __syncthreads();
    f32x4 nacc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) nacc[rb] = f32x4{in.r[rb][0], in.r[rb][1], in.r[rb][2], in.r[rb][3]};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
        bf16x8 shi, slo;
        split8(*reinterpret_cast<const f32x4*>(St + c * LS + 32 * kb + 8 * g),
               *reinterpret_cast<const f32x4*>(St + c * LS + 32 * kb + 8 * g + 4), shi, slo);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            bf16x8 phi, plo;
            split8(in.p[rb][kb][0], in.p[rb][kb][1], phi, plo);
            nacc[rb] = MF::mma(phi, shi, nacc[rb]);
            nacc[rb] = MF::mma(plo, shi, nacc[rb]);
            nacc[rb] = MF::mma(phi, slo, nacc[rb]);
        }
    }
    acc[0] = nacc[0];
    acc[1] = nacc[1];
    __syncthreads();
}

template <int DK, int DV>
// (s0 may be Sent itself: each element is read, then written with the same
// value, by one thread.)
__global__ __launch_bounds__(256) void scan_x3_kernel(const float* __restrict__ P, const float* __restrict__ R,
                                                      const float* s0, float* Sent, float* __restrict__ s_final,
                                                      int nseg, int nchain) {
    static_assert(DK == 128, "four waves of 32 state rows");
    constexpr int LS = DK + 4;
    __shared__ __align__(16) float St[16 * LS];
    const int tile = blockIdx.x / nchain;
    const size_t bh = blockIdx.x % nchain;
    const int l = lane_id(), w = wave_id();
    const int col0 = tile * 16;
    f32x4 acc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 32 * w + 16 * rb + 4 * (l >> 4) + e;
            acc[rb][e] = s0 ? s0[(bh * DK + row) * DV + col0 + (l & 15)] : 0.f;
        }
    ScanIn<DK, DV> a, b;
    scan_load<DK, DV>(a, P, R, 0, nchain, bh, col0, w, l);
    int j = 0;
    for (; j + 2 <= nseg; j += 2) {
        scan_load<DK, DV>(b, P, R, j + 1, nchain, bh, col0, w, l);
        scan_apply<DK, DV>(acc, a, Sent, St, j, nchain, bh, col0, w, l);
        scan_load<DK, DV>(a, P, R, min(j + 2, nseg - 1), nchain, bh, col0, w, l);
        scan_apply<DK, DV>(acc, b, Sent, St, j + 1, nchain, bh, col0, w, l);
    }
    if (j < nseg) scan_apply<DK, DV>(acc, a, Sent, St, j, nchain, bh, col0, w, l);
    if (s_final) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 32 * w + 16 * rb + 4 * (l >> 4) + e;
                s_final[(bh * DK + row) * DV + col0 + (l & 15)] = acc[rb][e];
            }
    }
}

// ---------------------------------------------------------------------------
// Host side.  Segments: one per chain (a single EXPAND pass from s0) when
// there are enough chains to fill the chip; otherwise about 1024 segments in
// all, of at least MIN_L chunks.
constexpr int MIN_L = 8;
constexpr int TARGET_WG = 256;
constexpr int FILL_CHAINS = 256;

struct Plan {
    int nseg, L;
    bool split;   // the first and last segments run as full expands (pipe_first_kernel, pipe_last_kernel)
    size_t p_off, r_off, e_off, tm_off, total;
};

// The pipelined kernels serve d_k = d_v = 128 unless KDA_PIPELINE=0 (the
// single-role fused kernels then run, for comparison).
static bool use_pipe() {
    static const bool on = [] {
        const char* e = getenv("KDA_PIPELINE");
        return !(e && e[0] == '0');
    }();
    return on;
}

// Uniform plan: nseg segments of L chunks (the last one shorter), composed,
// scanned and expanded.  With `split` (the pipelined kernels), a segmented
// plan of nseg segments becomes nseg + 1 of them, the first and last ones expanded directly (pipe_first_kernel,
// pipe_last_kernel), so each pass still runs nseg workgroups per chain.  The
// last segment, a full expand beside light expands, is made shorter: a full
// expand costs about 1.2x a light one per chunk, so L = NC / (nseg + 5/6)
// balances the second pass.
static Plan plan(int B, int T, int H, int DK, int DV, bool split = false) {
    Plan p{};
    const int NC = (T + C - 1) / C;
    const long nchain = (long)B * H;
    int nseg = 1;
    if (nchain < FILL_CHAINS && NC >= 2 * MIN_L) {
        const long want = (TARGET_WG + nchain - 1) / nchain;
        nseg = (int)(want < NC / MIN_L ? want : NC / MIN_L);
        if (nseg < 1) nseg = 1;
    }
    p.L = (NC + nseg - 1) / nseg;
    p.nseg = nseg > 1 ? (NC + p.L - 1) / p.L : 1;
    p.split = false;
    if (split && p.nseg > 1) {
        const int L = (int)((6L * NC + 6L * nseg + 4) / (6L * nseg + 5));   // ceil(NC / (nseg + 5/6))
        const int n = (NC + L - 1) / L;
        if (n >= 3) {
            p.L = L;
            p.nseg = n;
            p.split = true;
        }
    }
    p.p_off = p.r_off = p.e_off = p.tm_off = p.total = 0;
    if (p.nseg > 1) {
        p.r_off = (size_t)p.nseg * nchain * DK * DK * 4;
        p.e_off = p.r_off + (size_t)p.nseg * nchain * DK * DV * 4;
        p.tm_off = p.e_off + (size_t)p.nseg * nchain * DK * DV * 4;
        p.total = p.tm_off;
        // the pipelined path hands every chunk's T' from compose to expand
        if (DK == 128 && DV == 128 && use_pipe()) p.total += (size_t)nchain * NC * TM_ELEMS * 2;
    }
    return p;
}

template <class K>
static hipError_t set_lds(K kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int DK, int DV>
static hipError_t launch_scan(const ChunkArgs& a, const Plan& p, float* Pb, float* Rb, float* Eb) {
    const int nchain = a.B * a.H;
    if constexpr (DK == 128) {
        hipLaunchKernelGGL((scan_x3_kernel<DK, DV>), dim3((DV / 16) * nchain), dim3(256), 0, (hipStream_t)a.stream,
                           (const float*)Pb, (const float*)Rb, a.s0, Eb, a.s_final, p.nseg, nchain);
        return hipGetLastError();
    } else {
        return launch_seg_scan(Pb, Rb, a.s0, Eb, a.s_final, p.nseg, nchain, DK, DV, a.stream);
    }
}

// d_k = d_v = 128: compose (writing every chunk's T'), scan, and the light
// expand; one full expand pass when one segment per chain suffices.
template <bool GATED, bool SG>
static hipError_t launch_pipe_t(const ChunkArgs& a, const Plan& p) {
    const int NC = (a.T + C - 1) / C;
    const int nchain = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    const bf16 *q = (const bf16*)a.q, *k = (const bf16*)a.k, *v = (const bf16*)a.v, *z = (const bf16*)a.z,
               *beta = (const bf16*)a.beta, *gate = (const bf16*)a.gate;
    bf16* y = (bf16*)a.y;
    hipError_t err;
    if (p.nseg == 1) {
        // the epilogue is fused into the light expand only (segmented plans)
        if (GATED) return hipErrorInvalidValue;
        if ((err = set_lds(pipe_kernel<EXPAND, false, SG>, PLay<EXPAND>::LDS)) != hipSuccess) return err;
        hipLaunchKernelGGL((pipe_kernel<EXPAND, false, SG>), dim3(nchain), dim3(NTH), PLay<EXPAND>::LDS, st, q, k, v, z, beta,
                           a.g_min, a.T, a.H, NC, NC, nchain, a.s0, a.s_final, (float*)nullptr, (bf16*)a.o,
                           (bf16*)nullptr, (const bf16*)nullptr, 0.f, (bf16*)nullptr);
        return hipGetLastError();
    }
    unsigned char* ws = (unsigned char*)a.workspace;
    float* Pb = reinterpret_cast<float*>(ws + p.p_off);
    float* Rb = reinterpret_cast<float*>(ws + p.r_off);
    float* Eb = reinterpret_cast<float*>(ws + p.e_off);
    bf16* TM = reinterpret_cast<bf16*>(ws + p.tm_off);
    if (p.split) {
        // GATED: the first and last segments' outputs go to o, or else to
        // y's rows (same layout), and the epilogue kernel gates them there
        bf16* o_end = GATED && !a.o ? y : (bf16*)a.o;
        const size_t pslot = (size_t)nchain * 128 * 128;   // one segment's P, R or E (fp32)
        constexpr size_t LDS1 = PLay<EXPAND>::LDS > PLay<COMPOSE>::LDS ? PLay<EXPAND>::LDS : PLay<COMPOSE>::LDS;
        constexpr size_t LDS2 = PLay<EXPAND>::LDS > PLay<EXPAND_LITE>::LDS ? PLay<EXPAND>::LDS : PLay<EXPAND_LITE>::LDS;
        if ((err = set_lds(pipe_first_kernel<SG>, LDS1)) != hipSuccess) return err;
        hipLaunchKernelGGL((pipe_first_kernel<SG>), dim3((p.nseg - 1) * nchain), dim3(NTH), LDS1, st, q, k, v, z, beta,
                           a.g_min, a.T, a.H, NC, p.L, nchain, a.s0, Eb + pslot, Pb, Rb, o_end, TM);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        // entry states of segments 2 .. nseg-1 from that of segment 1 over
        // the transitions of segments 1 .. nseg-2
        hipLaunchKernelGGL((scan_x3_kernel<128, 128>), dim3(8 * nchain), dim3(256), 0, st, (const float*)(Pb + pslot),
                           (const float*)(Rb + pslot), (const float*)(Eb + pslot), Eb + pslot,
                           Eb + (size_t)(p.nseg - 1) * pslot, p.nseg - 2, nchain);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if ((err = set_lds(pipe_last_kernel<GATED, SG>, LDS2)) != hipSuccess) return err;
        hipLaunchKernelGGL((pipe_last_kernel<GATED, SG>), dim3((p.nseg - 1) * nchain), dim3(NTH), LDS2, st, q, k, v, z,
                           beta, a.g_min, a.T, a.H, NC, p.L, nchain, p.nseg, (const float*)Eb, a.s_final, (bf16*)a.o,
                           o_end, TM, gate, a.eps, y);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if constexpr (GATED) {
            // tokens [0, L C) and [(nseg - 1) L C, T) of every sequence
            const int t_a = min(a.T, p.L * C), t_b = (p.nseg - 1) * p.L * C;
            return launch_gate_ends(o_end, gate, a.eps, y, a.B, a.T, a.H, t_a, t_b, a.stream);
        }
        return hipSuccess;
    }
    if ((err = set_lds(pipe_kernel<COMPOSE, false, SG>, PLay<COMPOSE>::LDS)) != hipSuccess) return err;
    hipLaunchKernelGGL((pipe_kernel<COMPOSE, false, SG>), dim3(p.nseg * nchain), dim3(NTH), PLay<COMPOSE>::LDS, st, q, k, v, z,
                       beta, a.g_min, a.T, a.H, NC, p.L, nchain, (const float*)nullptr, Pb, Rb, (bf16*)nullptr, TM,
                       (const bf16*)nullptr, 0.f, (bf16*)nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_scan<128, 128>(a, p, Pb, Rb, Eb)) != hipSuccess) return err;
    if ((err = set_lds(pipe_kernel<EXPAND_LITE, GATED, SG>, PLay<EXPAND_LITE>::LDS)) != hipSuccess) return err;
    hipLaunchKernelGGL((pipe_kernel<EXPAND_LITE, GATED, SG>), dim3(p.nseg * nchain), dim3(NTH), PLay<EXPAND_LITE>::LDS,
                       st, q, k, v, z, beta, a.g_min, a.T, a.H, NC, p.L, nchain, (const float*)Eb, (float*)nullptr,
                       (float*)nullptr, (bf16*)a.o, TM, gate, a.eps, y);
    return hipGetLastError();
}
static hipError_t launch_pipe(const ChunkArgs& a, const Plan& p) {
    if (a.scalar_z) return a.gate ? hipErrorInvalidValue : launch_pipe_t<false, true>(a, p);
    return a.gate ? launch_pipe_t<true, false>(a, p) : launch_pipe_t<false, false>(a, p);
}

template <int DK, int DV>
static hipError_t launch_t(const ChunkArgs& a) {
    if constexpr (DK == 128 && DV == 128)
        if (use_pipe()) return launch_pipe(a, plan(a.B, a.T, a.H, DK, DV, true));
    const Plan p = plan(a.B, a.T, a.H, DK, DV);
    if (a.scalar_z) return hipErrorInvalidValue;   // only the pipelined kernels read a scalar gate
    const int NC = (a.T + C - 1) / C;
    const int nchain = a.B * a.H;
    hipStream_t st = (hipStream_t)a.stream;
    const bf16 *q = (const bf16*)a.q, *k = (const bf16*)a.k, *v = (const bf16*)a.v, *z = (const bf16*)a.z,
               *beta = (const bf16*)a.beta;
    typedef Lay<DK, DV, EXPAND> LE;
    typedef Lay<DK, DV, COMPOSE> LCm;
    hipError_t err;
    if ((err = set_lds(seg_kernel<DK, DV, EXPAND>, LE::LDS)) != hipSuccess) return err;
    if (p.nseg == 1) {
        hipLaunchKernelGGL((seg_kernel<DK, DV, EXPAND>), dim3(nchain), dim3(NTH), LE::LDS, st, q, k, v, z, beta,
                           a.g_min, a.T, a.H, NC, NC, nchain, a.s0, a.s_final, (float*)nullptr, (bf16*)a.o);
        return hipGetLastError();
    }
    unsigned char* ws = (unsigned char*)a.workspace;
    float* Pb = reinterpret_cast<float*>(ws + p.p_off);
    float* Rb = reinterpret_cast<float*>(ws + p.r_off);
    float* Eb = reinterpret_cast<float*>(ws + p.e_off);
    if ((err = set_lds(seg_kernel<DK, DV, COMPOSE>, LCm::LDS)) != hipSuccess) return err;
    hipLaunchKernelGGL((seg_kernel<DK, DV, COMPOSE>), dim3(p.nseg * nchain), dim3(NTH), LCm::LDS, st, q, k, v, z,
                       beta, a.g_min, a.T, a.H, NC, p.L, nchain, (const float*)nullptr, Pb, Rb, (bf16*)nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_scan<DK, DV>(a, p, Pb, Rb, Eb)) != hipSuccess) return err;
    hipLaunchKernelGGL((seg_kernel<DK, DV, EXPAND>), dim3(p.nseg * nchain), dim3(NTH), LE::LDS, st, q, k, v, z,
                       beta, a.g_min, a.T, a.H, NC, p.L, nchain, (const float*)Eb, (float*)nullptr, (float*)nullptr,
                       (bf16*)a.o);
    return hipGetLastError();
}

}  // namespace segk

size_t seg_workspace_bytes(int B, int T, int H, int dk, int dv) {
    // room for either plan (KDA_PIPELINE=0 selects the uniform one)
    const size_t u = segk::plan(B, T, H, dk, dv).total;
    const size_t s = dk == 128 && dv == 128 ? segk::plan(B, T, H, dk, dv, true).total : 0;
    return u > s ? u : s;
}

bool chunk_scalar_gate_native(int T, int dk, int dv, bool bf16, float g_min) {
    return bf16 && dk == 128 && dv == 128 && T > 0 && g_min >= CHUNK_G_MIN_LIMIT && segk::use_pipe();
}

bool chunk_gate_fused(int B, int T, int H, int dk, int dv, bool bf16) {
    return bf16 && dk == 128 && dv == 128 && segk::use_pipe() && segk::plan(B, T, H, dk, dv).nseg > 1;
}

hipError_t launch_chunk_seg(const ChunkArgs& a) {
    if (a.dk == 128 && a.dv == 128) return segk::launch_t<128, 128>(a);
    if (a.dk == 128 && a.dv == 64) return segk::launch_t<128, 64>(a);
    if (a.dk == 64 && a.dv == 128) return segk::launch_t<64, 128>(a);
    return segk::launch_t<64, 64>(a);
}

}  // namespace kda
