// bwd_chunk.hip -- kda_chunk_bwd: gradients of the KDA recurrence by 64-token
// chunks.  The pages give the forward only; this is the chain rule through
// the chunk form (Kimi Linear tech report, section 3.1 and appendix B,
// Eqs. 16-19, with the decay and readout of "KDA Recurrence").  Per chunk with
// entering state S, g = g_min sigmoid(z), G its chunk-local cumulative sum,
// Gam = e^G, Kg = K Gam, Kt = K / Gam, Kc = K e^{G_C - G}, Qg = Q Gam:
//   A = tril_-1(diag(beta) Kg Kt^T), M = tril(Qg Kt^T), T = (I + A)^{-1},
//   W = T diag(beta) Kg, U = T diag(beta) V, Vn = U - W S,
//   O = Qg S + M Vn,   S' = Diag(e^{G_C}) S + Kc^T Vn.
// With dO and dS' (the gradient of the state leaving the chunk) given:
//   dVn = M^T dO + Kc dS',                dS  = e^{G_C} dS' + Qg^T dO - W^T dVn,
//   dM  = tril(dO Vn^T),  dQg = dO S^T,   dKc = Vn dS'^T,   dW = -dVn S^T,
//   dT  = dW (diag(beta) Kg)^T + dVn (diag(beta) V)^T,
//   dBk = T^T dW, dBv = T^T dVn,          dA = tril_-1(-T^T dT T^T),
//   dV  = beta dBv,  dbeta = rowsum(dBv V + dBk Kg + dA Ab)  (Ab = Kg Kt^T),
//   dKg = beta dBk + (beta dA) Kt,  dKt = (beta dA)^T Kg + dM^T Qg,  dQg += dM Kt,
// then dQ = dQg Gam, dK = dKg Gam + dKt / Gam + dKc e^{G_C - G},
//   dG = dQ q + (dKg Gam - dKt / Gam - dKc e^{G_C - G}) k  (+ e^{G_C} rowsum(S dS')
//        + colsum(dKc e^{G_C - G} k) on the last row),
//   dg = reverse cumulative sum of dG,  dz = dg g_min sigmoid(z) (1 - sigmoid(z)).
//
// Kernels:
//  * the forward half (chunk.hip): the per-chunk operands of both directions,
//    then the chunk recurrence from S0 storing each chunk's S and Vn;
//  * dchain_kernel, one workgroup per (batch, head), one wave per 16 rows of
//    dS: the chunks in reverse, dS in MFMA accumulators; per chunk dVn and the products with S, Vn and
//    dS' (dQg, dW, dKc, dM and e^{G_C} rowsum(S dS')), written for the next
//    kernel;
//  * dintra_kernel, one 512-thread workgroup per chunk: everything else, on
//    fp32 MFMA.
//    The products whose terms carry e^{G_r - G_i} are evaluated per 16-row
//    block pair around reference rows m = 16R + 7, as in the forward, with
//    the cross-block factor applied as its square root twice.
#include <type_traits>

#include "chunk_layout.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwdc {

template <class E> __device__ __forceinline__ float dexp2(float x) { return __builtin_amdgcn_exp2f(x); }
template <> __device__ __forceinline__ float dexp2<float>(float x) { return exp2f(x); }

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr size_t a256(size_t x) { return (x + 255) / 256 * 256; }

// Per chunk, fp32, written by dchain_kernel for dintra_kernel.
template <int DK, int DV>
struct Ob {
    static constexpr size_t DVNT = 0;                       // (DV, C)  dVn^T
    static constexpr size_t DQGT = DVNT + (size_t)DV * C;   // (DK, C)  (dO S^T)^T
    static constexpr size_t DWT = DQGT + (size_t)DK * C;    // (DK, C)  (-dVn S^T)^T
    static constexpr size_t DKCT = DWT + (size_t)DK * C;    // (DK, C)  (Vn dS'^T)^T
    static constexpr size_t DMT = DKCT + (size_t)DK * C;    // (C, C)   tril(dO Vn^T)^T
    static constexpr size_t DGC = DMT + (size_t)C * C;      // (DK)     e^{G_C} rowsum(S dS')
    static constexpr size_t END = DGC + DK;
    static constexpr size_t BYTES = END * 4;
};

// Per chunk, bf16 tokens: bf16 products, each stored in the orientation the
// per-chunk kernel contracts it in (offsets in bf16 elements; each matrix in
// 16 x 16 tiles, see tix), then the fp32 e^{G_C} rowsum(S dS').
// NP = -tril_-1(dVn Vn^T), which with dT T^T = dVn Vn^T (I + A)^T T^T =
// dVn Vn^T gives dA = tril_-1(T^T NP).
template <int DK, int DV>
struct ObH {
    static constexpr size_t DVNT = 0;                      // (DV, C)  dVn^T
    static constexpr size_t DWT = DVNT + (size_t)DV * C;   // (DK, C)  (-dVn S^T)^T
    static constexpr size_t DQG = DWT + (size_t)DK * C;    // (C, DK)  dO S^T
    static constexpr size_t DKC = DQG + (size_t)C * DK;    // (C, DK)  Vn dS'^T
    static constexpr size_t NPT = DKC + (size_t)C * DK;    // (C, C)   NP^T
    static constexpr size_t DM = NPT + (size_t)C * C;      // (C, C)   tril(dO Vn^T)
    static constexpr size_t DMT = DM + (size_t)C * C;      // (C, C)   its transpose
    static constexpr size_t END = DMT + (size_t)C * C;
    static constexpr size_t DGC_BYTE = END * 2;            // (DK) fp32
    static constexpr size_t BYTES = DGC_BYTE + DK * 4;
    static_assert(BYTES % 16 == 0, "16-byte aligned chunk blocks");
};

// Element (r, c) of an ObH matrix with ncol columns: 16 x 16 tiles in
// row-major tile order, each tile row-major, so that a wave's 16 x 16 MFMA
// result (4 consecutive columns per lane) is one contiguous 512-byte store
// and a fragment read (4 or 8 consecutive columns of 16 rows) stays inside a
// tile's rows.
__device__ __forceinline__ size_t tix(int r, int c, int ncol) {
    return ((size_t)(r >> 4) * (ncol >> 4) + (c >> 4)) * 256 + (r & 15) * 16 + (c & 15);
}

template <class CT, int DK, int DV>
constexpr size_t ob_bytes() {
    if constexpr (std::is_same<CT, bf16>::value) return ObH<DK, DV>::BYTES;
    return Ob<DK, DV>::BYTES;
}

struct Lay {
    size_t fws, bws, st, vn, ob, total;
};

template <class CT, int DK, int DV>
Lay lay_t(int B, int T, int H) {
    const size_t nchunk = (size_t)B * H * (((size_t)T + C - 1) / C);
    Lay lo{};
    lo.fws = 0;
    lo.bws = a256(nchunk * Ws<CT, DK, DV>::BYTES);
    lo.st = lo.bws + a256(nchunk * WsB<CT, DK, DV>::BYTES);
    lo.vn = lo.st + a256(nchunk * DK * DV * sizeof(CT));
    lo.ob = lo.vn + a256(nchunk * C * DV * sizeof(CT));
    lo.total = lo.ob + nchunk * ob_bytes<CT, DK, DV>();
    return lo;
}

// Sum over the 16 lanes of a DPP row, in every lane: quad swaps, then the
// half-row and row mirrors.
__device__ __forceinline__ float sum16(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

// A workgroup barrier for LDS hand-offs that leaves global loads in flight
// (__syncthreads would wait for every one of them): lgkmcnt(0) completes
// this wave's LDS accesses, and the wavefront-scope fences keep the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Two adjacent 16-channel tiles P (channels c .. c + 15) and Q (c + 16 ..
// c + 31) in the layout of a 16x16 MFMA result (lane lr + 16 lg: row lr,
// channels 4 lg .. 4 lg + 3 of its tile), rearranged for row-contiguous
// stores: lane 8 r + j of lo holds row r and of hi row r + 8, channels
// c + 4 j .. c + 4 j + 3, so that one store instruction covers 8 rows of 128
// contiguous bytes rather than 16 rows of 64.  A rotate by 8 lanes within
// each 16-lane DPP row first brings row r + 8 of one tile beside row r of
// the other; ds_bpermute then gathers.
__device__ __forceinline__ void pair_rows(const f32x4& P, const f32x4& Q, f32x4& lo, f32x4& hi) {
    const int l = lane_id(), lr = l & 15, r = l >> 3, j = l & 7;
    const int src = ((j & 3) * 16 + r + 8 * (j >> 2)) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // the element into a scalar first: clang bit-casts a subscripted vector
        // element as element 0
        const float pe = P[e], qe = Q[e];
        const int p = __builtin_bit_cast(int, pe), q = __builtin_bit_cast(int, qe);
        const int pr = __builtin_amdgcn_mov_dpp(p, 0x128, 0xF, 0xF, false);
        const int qr = __builtin_amdgcn_mov_dpp(q, 0x128, 0xF, 0xF, false);
        lo[e] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, lr < 8 ? p : qr));
        hi[e] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, lr < 8 ? pr : q));
    }
}

// ---------------------------------------------------------------------------
// Reverse chunk recurrence of one chain (b, h), all d_v columns: one wave per
// 16 rows of dS (d_k / 16 waves).  dS rows of wave w: 16w + 4(l/16) + e,
// columns ct*16 + l%16.  The chunk's token-row products are split over the
// waves as row block X = w % 4 times column group w / 4.
// ---------------------------------------------------------------------------
template <class E, int DK, int DV>
struct DChain {
    typedef typename Compute<E>::type CT;
    typedef Mfma<CT> MF;
    static constexpr int NW = DK / 16, NTH = 64 * NW, NCG = NW / 4;   // column groups of the token-row products
    static constexpr int KS = MF::KSTEP, NT = DV / 16;
    static constexpr int LC = C + 8, LDK = DK + 8, LDV = DV + 8;
    static constexpr size_t OFF_DOT = 0;                                                  // [DV][LC]  dO^T
    static constexpr size_t OFF_DST = OFF_DOT + align16((size_t)DV * LC * sizeof(CT));   // [DV][LDK] dS^T
    static constexpr size_t OFF_DSR = OFF_DST + align16((size_t)DV * LDK * sizeof(CT));  // [DK][LDV] dS
    static constexpr size_t OFF_DVT = OFF_DSR + align16((size_t)DK * LDV * sizeof(CT));  // [DV][LC]  -dVn^T
    static constexpr size_t OFF_DVR = OFF_DVT + align16((size_t)DV * LC * sizeof(CT));   // [C][LDV]  -dVn
    // bf16: the chunk's entering state S, staged by asynchronous global->LDS
    // loads one chunk ahead; rows of DV elements in 16-byte groups, group g of
    // row r at position g ^ (r mod DV/8), so a fragment read (16 rows, one
    // group) touches 16 distinct positions
    static constexpr bool SL = std::is_same<CT, bf16>::value;
    static constexpr size_t OFF_S = OFF_DVR + align16((size_t)C * LDV * sizeof(CT));     // [DK][DV]  S
    static constexpr size_t LDS = OFF_S + (SL ? (size_t)DK * DV * 2 : 0);
    static_assert(LDS <= 160 * 1024, "reverse chain LDS budget");
    static_assert(!SL || ((size_t)DK * DV * 2) % (1024 * NW) == 0, "whole 1 KB loads per wave");
    static_assert(NW % 4 == 0 && NT % NCG == 0 && (DK / 16) % NCG == 0 && (C / 16) % NCG == 0, "wave split");
};

// One chunk's entering state S (DK x DV bf16) into LDS by asynchronous
// global->LDS loads: wave instruction i fills bytes 1024 i .. 1024 i + 1023;
// group g of row r lands at position g ^ (r mod DV/8) of its row.
template <int DK, int DV, int NW>
__device__ __forceinline__ void stage_state(const bf16* __restrict__ src, unsigned char* lds) {
    constexpr int SG = DV / 8, PER_WAVE = DK * DV * 2 / 1024 / NW;
    const int w = wave_id(), l = lane_id();
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int ins = w * PER_WAVE + i, byte = ins * 1024 + 16 * l;
        const int r = byte / (DV * 2), p = (byte % (DV * 2)) / 16, g = p ^ (r & (SG - 1));
        __builtin_amdgcn_global_load_lds(src + (size_t)r * DV + g * 8, lds + ins * 1024, 16, 0, 0);
    }
}
template <int DK, int DV, int NW>
__device__ __forceinline__ void stage_state(const float*, unsigned char*) {}   // fp32: S is read from memory

template <class E, int DK, int DV>
__global__ __launch_bounds__(DK * 4) void dchain_kernel(const E* __restrict__ dout, const float* __restrict__ ds_final,
                                                        float* __restrict__ ds0, int T, int H, int NC,
                                                        const unsigned char* __restrict__ fws,
                                                        const unsigned char* __restrict__ bws,
                                                        const typename Compute<E>::type* __restrict__ states,
                                                        const typename Compute<E>::type* __restrict__ vn,
                                                        unsigned char* __restrict__ obuf) {
    typedef DChain<E, DK, DV> L;
    typedef typename L::CT CT;
    typedef typename L::MF MF;
    typedef Ws<CT, DK, DV> WL;
    typedef WsB<CT, DK, DV> WB;
    typedef Ob<DK, DV> OL;
    typedef ObH<DK, DV> OH;
    constexpr bool H16 = std::is_same<CT, bf16>::value;   // bf16 products for dintra16_kernel
    constexpr int KS = L::KS, NT = L::NT, LC = L::LC, LDK = L::LDK, LDV = L::LDV, NTH = L::NTH, NCG = L::NCG;
    constexpr int VE = 16 / sizeof(CT);   // elements per 16-byte access
    extern __shared__ __align__(16) unsigned char smem[];
    CT* dOT = reinterpret_cast<CT*>(smem + L::OFF_DOT);
    CT* dST = reinterpret_cast<CT*>(smem + L::OFF_DST);
    CT* dSR = reinterpret_cast<CT*>(smem + L::OFF_DSR);
    CT* dVT = reinterpret_cast<CT*>(smem + L::OFF_DVT);
    CT* dVR = reinterpret_cast<CT*>(smem + L::OFF_DVR);
    CT* Ss = reinterpret_cast<CT*>(smem + L::OFF_S);

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int X = w & 3, cg = w >> 2;         // token-row block and column group of this wave
    const size_t bh = blockIdx.x;
    const int bb = (int)(bh / H), hh = (int)(bh % H);
    constexpr int SG = DV / 8;                // 16-byte groups per row of S
    auto issue_s = [&](int m) { stage_state<DK, DV, L::NW>(states + (bh * NC + m) * DK * DV, smem + L::OFF_S); };
    // fragment (rows row0 + l%16, columns k0 + 8(l/16) ..) and element reads of the staged S
    auto s_frag = [&](int row0, int k0, int l) -> typename MF::frag {
        const int r = row0 + (l & 15), g = k0 / 8 + (l >> 4);
        return *reinterpret_cast<const typename MF::frag*>(Ss + r * DV + ((g ^ (r & (SG - 1))) << 3));
    };
    auto s_elem = [&](int r, int c) -> float {
        return to_f32(Ss[r * DV + ((((c >> 3) ^ (r & (SG - 1))) << 3) | (c & 7))]);
    };
    if constexpr (L::SL) issue_s(NC - 1);
    // dO rows of chunk m into registers, zero past the end of the sequence
    constexpr int NU = C * DV / VE / NTH;
    static_assert(NU * VE * NTH == C * DV, "whole dO rows per thread");
    // (raw 16-byte vectors: rows past the end are zeroed when staged, so the
    // loads are not waited for here)
    u32x4 dov[NU];
    auto load_do = [&](int m, int tid) {
        const int valid_m = min(C, T - m * C);
        const E* dob_m = dout + (((size_t)bb * T + (size_t)m * C) * H + hh) * DV;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = tid + i * NTH, r = u % C, j0 = (u / C) * VE;   // consecutive lanes: consecutive tokens
            dov[i] = *reinterpret_cast<const u32x4*>(dob_m + (size_t)min(r, valid_m - 1) * H * DV + j0);
        }
    };
    load_do(NC - 1, tid);
    const int srow = w * 16 + 4 * (l >> 4);   // first dS row of this lane

    f32x4 accD[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const int col = ct * 16 + (l & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) accD[ct][e] = ds_final ? ds_final[(bh * DK + srow + e) * DV + col] : 0.f;
    }
    auto store_ds = [&](int l, int srow) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int col = ct * 16 + (l & 15);
            store4<CT>(dST + col * LDK + srow, accD[ct]);
#pragma unroll
            for (int e = 0; e < 4; ++e) dSR[(srow + e) * LDV + col] = from_f32<CT>(accD[ct][e]);
        }
    };
    store_ds(l, srow);

    for (int n = NC - 1; n >= 0; --n) {
        // lane-derived addresses are recomputed in every chunk instead of
        // being held in registers across the loop
        const int l = opaque(lane_id()), tid = opaque((int)threadIdx.x);
        const int srow = w * 16 + 4 * (l >> 4);
        const int valid = min(C, T - n * C);
        const size_t cid = bh * NC + n;
        const unsigned char* fb = fws + cid * WL::BYTES;
        const CT* bk = reinterpret_cast<const CT*>(bws + cid * WB::BYTES);
        const CT* Sn = states + cid * DK * DV;
        const CT* Vn = vn + cid * C * DV;
        float* ob = reinterpret_cast<float*>(obuf + cid * ob_bytes<CT, DK, DV>());
        bf16* obh = reinterpret_cast<bf16*>(ob);
        const E* dob = dout + (((size_t)bb * T + (size_t)n * C) * H + hh) * DV;   // row r at r * H * DV
        const size_t rs = (size_t)H * DV;

        // this wave's M^T and Kc rows (token block X) for dVn; then, for the
        // products after dVn, dO rows 16X.. (zero past the end) and Vn rows
        // 16X.. as A operands, and the Vn rows of this wave's dM blocks: all
        // issued first, so that they arrive while dO^T is staged and dVn runs
        typename MF::frag mtf[C / KS], kcf[DK / KS];
#pragma unroll
        for (int kk = 0; kk < C / KS; ++kk) mtf[kk] = load_frag<CT>(bk + WB::MT, C, X * 16, kk * KS, l);
        // e^{G_C} of this wave's rows, for the row sums and the dS update
        const f32x4 eg = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(fb + WL::END * sizeof(CT)) + srow);
#pragma unroll
        for (int kk = 0; kk < DK / KS; ++kk) kcf[kk] = load_frag<CT>(bk + WB::KC, DK, X * 16, kk * KS, l);
        constexpr int NKK = DV / KS, NIB = C / 16 / NCG;
        typename MF::frag dof[NKK], vf[NKK], fvm[NIB][NKK];
        {
            const int r = X * 16 + (l & 15);
            const bool ok = r < valid;
            // the row address is clamped to the last token (in bounds); rows
            // past the end are zeroed
            const CT* drow = reinterpret_cast<const CT*>(dob + (size_t)min(r, valid - 1) * rs) + (l >> 4) * MF::KPL;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                dof[kk] = *reinterpret_cast<const typename MF::frag*>(drow + kk * KS);
                if (!ok) dof[kk] = typename MF::frag{};
                vf[kk] = load_frag<CT>(Vn, DV, X * 16, kk * KS, l);
#pragma unroll
                for (int u = 0; u < NIB; ++u) fvm[u][kk] = load_frag<CT>(Vn, DV, (cg * NIB + u) * 16, kk * KS, l);
            }
        }

        // dO^T into LDS (rows loaded into registers during the previous chunk)
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = tid + i * NTH, r = u % C, j0 = (u / C) * VE;
            CT vals[VE];
            __builtin_memcpy(vals, &dov[i], 16);
#pragma unroll
            for (int x = 0; x < VE; ++x) dOT[(j0 + x) * LC + r] = r < valid ? vals[x] : from_f32<CT>(0.f);
        }
        lds_barrier();
        // the next chunk's dO rows, a whole chunk ahead of their staging
        if (n > 0) load_do(n - 1, tid);

        // dVn = M^T dO + Kc dS' (token rows 16X.., this wave's column group)
        constexpr int NTG = NT / NCG;
        f32x4 accV[NTG];
#pragma unroll
        for (int ct = 0; ct < NTG; ++ct) accV[ct] = zero4();
#pragma unroll
        for (int kk = 0; kk < C / KS; ++kk) {
#pragma unroll
            for (int ct = 0; ct < NTG; ++ct)
                accV[ct] = MF::mma(mtf[kk], load_frag<CT>(dOT, LC, (cg * NTG + ct) * 16, kk * KS, l), accV[ct]);
        }
#pragma unroll
        for (int kk = 0; kk < DK / KS; ++kk) {
#pragma unroll
            for (int ct = 0; ct < NTG; ++ct)
                accV[ct] = MF::mma(kcf[kk], load_frag<CT>(dST, LDK, (cg * NTG + ct) * 16, kk * KS, l), accV[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < NTG; ++ct) {
            const int col = (cg * NTG + ct) * 16 + (l & 15), row = X * 16 + 4 * (l >> 4);
            if constexpr (H16)
                store4<bf16>(obh + OH::DVNT + tix(col, row, C), accV[ct]);
            else
                *reinterpret_cast<f32x4*>(ob + OL::DVNT + (size_t)col * C + row) = accV[ct];
            store4<CT>(dVT + col * LC + row, -accV[ct]);
#pragma unroll
            for (int e = 0; e < 4; ++e) dVR[(row + e) * LDV + col] = from_f32<CT>(-accV[ct][e]);
        }
        if constexpr (L::SL) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's S loads have landed
        __syncthreads();

        // dQg = dO S^T, dW = -dVn S^T and dKc = Vn dS'^T (rows 16X.., this
        // wave's group of d_k column tiles)
        constexpr int NCB = DK / 16 / NCG;
        // operand fragments from LDS, issued one column block ahead of their
        // MFMAs (double-buffered); -dVn's rows are the same for every block
        typename MF::frag fvr[NKK], fsb[2][NKK], fdb[2][NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) fvr[kk] = load_frag<CT>(dVR, LDV, X * 16, kk * KS, l);
        auto load_cb = [&](int u, typename MF::frag (&fs)[NKK], typename MF::frag (&fd)[NKK]) {
            const int cb = cg * NCB + u;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if constexpr (L::SL)
                    fs[kk] = s_frag(cb * 16, kk * KS, l);
                else
                    fs[kk] = load_frag<CT>(Sn, DV, cb * 16, kk * KS, l);
                fd[kk] = load_frag<CT>(dSR, LDV, cb * 16, kk * KS, l);
            }
        };
        load_cb(0, fsb[0], fdb[0]);
#pragma unroll
        for (int u = 0; u < NCB; ++u) {
            const int cb = cg * NCB + u;
            if (u + 1 < NCB) load_cb(u + 1, fsb[(u + 1) & 1], fdb[(u + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);   // the next block's reads stay ahead of these MFMAs
            const typename MF::frag(&fs)[NKK] = fsb[u & 1];
            const typename MF::frag(&fd)[NKK] = fdb[u & 1];
            f32x4 accQ = zero4(), accW = zero4(), accK = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                accW = MF::mma(fvr[kk], fs[kk], accW);
                if constexpr (H16) {   // (channel, token) orientation: rows of dO S^T and Vn dS'^T
                    accQ = MF::mma(fs[kk], dof[kk], accQ);
                    accK = MF::mma(fd[kk], vf[kk], accK);
                } else {
                    accQ = MF::mma(dof[kk], fs[kk], accQ);
                    accK = MF::mma(vf[kk], fd[kk], accK);
                }
            }
            if constexpr (H16) {
                store4<bf16>(obh + OH::DQG + tix(X * 16 + (l & 15), cb * 16 + 4 * (l >> 4), DK), accQ);
                store4<bf16>(obh + OH::DWT + tix(cb * 16 + (l & 15), X * 16 + 4 * (l >> 4), C), accW);
                store4<bf16>(obh + OH::DKC + tix(X * 16 + (l & 15), cb * 16 + 4 * (l >> 4), DK), accK);
            } else {
                const size_t off = (size_t)(cb * 16 + (l & 15)) * C + X * 16 + 4 * (l >> 4);
                *reinterpret_cast<f32x4*>(ob + OL::DQGT + off) = accQ;
                *reinterpret_cast<f32x4*>(ob + OL::DWT + off) = accW;
                *reinterpret_cast<f32x4*>(ob + OL::DKCT + off) = accK;
            }
        }
        // dM = tril(dO Vn^T) (rows r, columns i), stored transposed
#pragma unroll
        for (int u = 0; u < NIB; ++u) {
            const int ib = cg * NIB + u;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) acc = MF::mma(dof[kk], fvm[u][kk], acc);
            const int i = ib * 16 + (l & 15), r0 = X * 16 + 4 * (l >> 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = (i <= r0 + e) ? acc[e] : 0.f;
            if constexpr (H16) {
                // dM row-major (rows 16X + l%16, columns ib*16 + 4(l/16) + e) and
                // NP = -tril_-1(dVn Vn^T), stored transposed
                f32x4 accR = zero4(), accP = zero4();
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    accR = MF::mma(fvm[u][kk], dof[kk], accR);
                    accP = MF::mma(fvr[kk], fvm[u][kk], accP);
                }
                const int r = X * 16 + (l & 15), i0 = ib * 16 + 4 * (l >> 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    accR[e] = (i0 + e <= r) ? accR[e] : 0.f;
                    accP[e] = (i < r0 + e) ? accP[e] : 0.f;
                }
                store4<bf16>(obh + OH::DMT + tix(i, r0, C), acc);
                store4<bf16>(obh + OH::DM + tix(r, i0, C), accR);
                store4<bf16>(obh + OH::NPT + tix(i, r0, C), accP);
            } else {
                *reinterpret_cast<f32x4*>(ob + OL::DMT + (size_t)i * C + r0) = acc;
            }
        }
        // (Q e^G)^T and W^T rows of this wave for the dS update, loaded here
        // so that they arrive during the row sums
        typename MF::frag aqf[C / KS], awf[C / KS];
#pragma unroll
        for (int kk = 0; kk < C / KS; ++kk) {
            aqf[kk] = load_frag<CT>(bk + WB::QGT, C, w * 16, kk * KS, l);
            awf[kk] = load_frag<CT>(bk + WB::WT, C, w * 16, kk * KS, l);
        }
        // e^{G_C} rowsum(S dS'), rows of this wave
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float sacc = 0.f;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                if constexpr (L::SL)
                    sacc += accD[ct][e] * s_elem(srow + e, ct * 16 + (l & 15));
                else
                    sacc += accD[ct][e] * to_f32(Sn[(size_t)(srow + e) * DV + ct * 16 + (l & 15)]);
            }
            sacc = sum16(sacc);
            if ((l & 15) == 0) {
                if constexpr (H16)
                    reinterpret_cast<float*>(obuf + cid * OH::BYTES + OH::DGC_BYTE)[srow + e] = sacc * eg[e];
                else
                    ob[OL::DGC + srow + e] = sacc * eg[e];
            }
        }
        // dS <- e^{G_C} dS' + Qg^T dO - W^T dVn
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) accD[ct] *= eg;
#pragma unroll
        for (int kk = 0; kk < C / KS; ++kk) {
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                accD[ct] = MF::mma(aqf[kk], load_frag<CT>(dOT, LC, ct * 16, kk * KS, l), accD[ct]);
                accD[ct] = MF::mma(awf[kk], load_frag<CT>(dVT, LC, ct * 16, kk * KS, l), accD[ct]);
            }
        }
        lds_barrier();   // this chunk's reads of dO^T, dS, dVn and S in LDS are done
        if constexpr (L::SL) {
            if (n > 0) issue_s(n - 1);   // lands before the next chunk's products (the barrier after its dVn waits)
        }
        store_ds(l, srow);
    }
    if (ds0) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int col = ct * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) ds0[(bh * DK + srow + e) * DV + col] = accD[ct][e];
        }
    }
}

// ---------------------------------------------------------------------------
// Per-chunk gradients: 512 threads, fp32 MFMA (16x16x4).  Wave w owns token
// rows 16X..16X+15 (X = w % 4) and one half of the d_k columns (w / 4) of the
// C x d_k results dQ, dK and dG, held in registers in the accumulator layout
// (rows 16X + 4(l/16) + e, column ct*16 + l%16).
// ---------------------------------------------------------------------------
template <class E, int DK, int DV>
struct DIntra {
    static constexpr int NTH = 512, NW = 8;
    static constexpr int CP = DK / 2, NPART = NTH / CP, RP = C / NPART;
    static constexpr int NCT = DK / 16, NCTH = NCT / 2, NVTH = DV / 32;   // column tiles per half
    static constexpr int DKP = DK + 4, LA = C + 4;
    static constexpr int NCAR = NPART > NW ? NPART : NW;
    static constexpr int DVP = DV + 4;
    static constexpr size_t OFF_G = 0;                                  // [C][DKP] G (log2 units), then dG
    static constexpr size_t OFF_K = OFF_G + (size_t)C * DKP * 4;        // [C][DKP] k (token precision)
    static constexpr size_t OFF_A = OFF_K + align16((size_t)C * DKP * sizeof(E));   // [C][LA] Ab, then q
    static constexpr size_t OFF_T = OFF_A + (size_t)C * LA * 4;         // [C][LA]  T
    static constexpr size_t OFF_S1 = OFF_T + (size_t)C * LA * 4;        // [C][LA]  dT, then beta dA
    static constexpr size_t OFF_S2 = OFF_S1 + (size_t)C * LA * 4;       // [C][LA]  v, then dT T^T, then dM
    // q is staged over Ab once Ab is dead, where it fits; else read from memory
    static constexpr bool QLDS = (size_t)C * DKP * sizeof(E) <= (size_t)C * LA * 4;
    static_assert((size_t)C * DVP * sizeof(E) <= (size_t)C * LA * 4, "v staged over S2");
    static constexpr size_t OFF_X = OFF_S2 + (size_t)C * LA * 4;        // [3][16][16]
    static constexpr size_t OFF_DSC = OFF_X + 3 * SUB * SUB * 4;        // [6][DK]
    static constexpr size_t OFF_GM = OFF_DSC + 6 * DK * 4;              // [5][DK] G_m(R), G_C
    static constexpr size_t OFF_CAR = OFF_GM + 5 * DK * 4;              // [NCAR][DK]
    static constexpr size_t OFF_BET = OFF_CAR + (size_t)NCAR * DK * 4;  // [C]
    static constexpr size_t OFF_DB = OFF_BET + C * 4;                   // [2][C] dbeta, per column half
    static constexpr size_t LDS = OFF_DB + 2 * C * 4;
    static_assert(LDS <= 160 * 1024, "per-chunk gradient LDS budget");
    static_assert(RP % 2 == 0 && 16 % RP == 0 && NCT % 2 == 0 && DV % 32 == 0, "tiling");
};

// Block pairs (R, I), I <= R, of the 64 x 64 lower triangle, by wave.
__constant__ int kPairsB[8][2][2] = {{{0, 0}, {1, 0}}, {{1, 1}, {2, 0}}, {{2, 1}, {-1, -1}}, {{2, 2}, {-1, -1}},
                                     {{3, 0}, {-1, -1}}, {{3, 1}, {-1, -1}}, {{3, 2}, {-1, -1}},
                                     {{3, 3}, {-1, -1}}};

__device__ __forceinline__ int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }   // I < R

__device__ __forceinline__ void upper_block(int p, int& R, int& I) {   // p = 0..5, I > R
    R = p < 3 ? 0 : (p < 5 ? 1 : 2);
    I = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
}

template <class E, int DK, int DV>
__global__ __launch_bounds__(512) void dintra_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                     const E* __restrict__ v, const E* __restrict__ z,
                                                     const E* __restrict__ beta, float g_min, int T, int H, int NC,
                                                     const unsigned char* __restrict__ obuf, float* __restrict__ dq,
                                                     float* __restrict__ dk, float* __restrict__ dvo,
                                                     float* __restrict__ dz, float* __restrict__ dbeta) {
    typedef DIntra<E, DK, DV> L;
    typedef Ob<DK, DV> OL;
    constexpr int NTH = L::NTH, RP = L::RP, DKP = L::DKP, LA = L::LA, NCTH = L::NCTH, NVTH = L::NVTH;
    constexpr float LOG2E = 1.4426950408889634f;
    extern __shared__ __align__(16) unsigned char smem[];
    float* Gs = reinterpret_cast<float*>(smem + L::OFF_G);
    E* Ks = reinterpret_cast<E*>(smem + L::OFF_K);
    E* Vs = reinterpret_cast<E*>(smem + L::OFF_S2);   // until dT T^T is formed
    E* Qs = reinterpret_cast<E*>(smem + L::OFF_A);    // once Ab is dead (QLDS)
    constexpr int DVP = L::DVP;
    float* As = reinterpret_cast<float*>(smem + L::OFF_A);
    float* Ts = reinterpret_cast<float*>(smem + L::OFF_T);
    float* S1 = reinterpret_cast<float*>(smem + L::OFF_S1);
    float* S2 = reinterpret_cast<float*>(smem + L::OFF_S2);
    float* Xs = reinterpret_cast<float*>(smem + L::OFF_X);
    float* dsc = reinterpret_cast<float*>(smem + L::OFF_DSC);
    float* gm = reinterpret_cast<float*>(smem + L::OFF_GM);
    float* car = reinterpret_cast<float*>(smem + L::OFF_CAR);
    float* bet = reinterpret_cast<float*>(smem + L::OFF_BET);
    float* dbt = reinterpret_cast<float*>(smem + L::OFF_DB);

    const int n = blockIdx.x, hh = blockIdx.y, bb = blockIdx.z;
    const int valid = min(C, T - n * C), last = valid - 1;
    const size_t row0 = ((size_t)bb * T + (size_t)n * C) * H + hh;   // token row of chunk row 0
    const float* ob = reinterpret_cast<const float*>(obuf + (((size_t)bb * H + hh) * NC + n) * OL::BYTES);
    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int lr = l & 15, lg = l >> 4;
    const int X = w & 3, hf = w >> 2;            // row block and column half of this wave
    const int rowA = X * 16 + lr;                 // A-operand row of this lane
    const int rowD = X * 16 + 4 * lg;             // first accumulator row of this lane

    // ---- gate, chunk-local scan (log2 units), k into LDS
    {
        const int c0 = 2 * (tid % L::CP), part = tid / L::CP, r0 = part * RP;
        const float kg2 = g_min * LOG2E;
        float G[RP][2];
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
            const size_t off = (row0 + (size_t)min(r, last) * H) * DK + c0;
            const typename Pair<E>::type zz = load2<E>(z + off), kk = load2<E>(k + off);
            const bool ok = r < valid;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float g2 = kg2 * __builtin_amdgcn_rcpf(1.0f + dexp2<E>(-LOG2E * to_f32(zz[j])));
                G[i][j] = ok ? g2 : 0.f;
                Ks[r * DKP + c0 + j] = ok ? kk[j] : from_f32<E>(0.f);
            }
            s0 += G[i][0];
            s1 += G[i][1];
            G[i][0] = s0;
            G[i][1] = s1;
        }
        car[part * DK + c0] = s0;
        car[part * DK + c0 + 1] = s1;
        if (tid < C) {
            bet[tid] = tid < valid ? to_f32(beta[row0 + (size_t)tid * H]) : 0.f;
            dbt[tid] = 0.f;
            dbt[C + tid] = 0.f;
        }
        __syncthreads();
        float cr[2] = {0.f, 0.f}, gC[2] = {0.f, 0.f};
#pragma unroll
        for (int p = 0; p < L::NPART; ++p)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float t = car[p * DK + c0 + j];
                if (p < part) cr[j] += t;
                gC[j] += t;
            }
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float g = G[i][j] + cr[j];
                Gs[r * DKP + c0 + j] = g;
                if ((r & 15) == 7) gm[(r >> 4) * DK + c0 + j] = g;
            }
        }
        if (part == 0) {
            gm[4 * DK + c0] = gC[0];
            gm[4 * DK + c0 + 1] = gC[1];
        }
        __syncthreads();
    }
    for (int idx = tid; idx < 6 * DK; idx += NTH) {
        const int p = idx / DK, cc = idx % DK;
        const int R = p < 1 ? 1 : (p < 3 ? 2 : 3);
        const int I = p - R * (R - 1) / 2;
        dsc[idx] = dexp2<E>(0.5f * (gm[R * DK + cc] - gm[I * DK + cc]));
    }
    __syncthreads();

    // ---- Ab = tril_-1(Kg Kt^T) per block pair; upper blocks of Ab and T zero
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
        const int R = kPairsB[w][jp][0], I = kPairsB[w][jp][1];
        if (R < 0) break;
        const float* dv = dsc + (I < R ? pair_index(R, I) : 0) * DK;
        const int ra = R * 16 + lr, ib = I * 16 + lr;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += 4) {
            const int c = kk + lg;
            const float a = to_f32(Ks[ra * DKP + c]) * dexp2<E>(Gs[ra * DKP + c] - gm[R * DK + c]);
            float b = to_f32(Ks[ib * DKP + c]) * dexp2<E>(gm[I * DK + c] - Gs[ib * DKP + c]);
            if (I < R) b = (b * dv[c]) * dv[c];
            acc = mma4(a, b, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = R * 16 + 4 * lg + e, i = I * 16 + lr;
            As[r * LA + i] = i < r ? acc[e] : 0.f;
        }
    }
    for (int idx = tid; idx < 6 * SUB * SUB; idx += NTH) {
        int R, I;
        upper_block(idx / (SUB * SUB), R, I);
        const int e = idx % (SUB * SUB);
        As[(R * SUB + e / SUB) * LA + I * SUB + e % SUB] = 0.f;
        Ts[(R * SUB + e / SUB) * LA + I * SUB + e % SUB] = 0.f;
    }
    // v into LDS (zero past the end), two elements per access
    for (int idx = tid; idx < C * DV / 2; idx += NTH) {
        const int r = idx / (DV / 2), j = 2 * (idx % (DV / 2));
        const typename Pair<E>::type vv = load2<E>(v + (row0 + (size_t)min(r, last) * H) * DV + j);
        Vs[r * DVP + j] = r < valid ? vv[0] : from_f32<E>(0.f);
        Vs[r * DVP + j + 1] = r < valid ? vv[1] : from_f32<E>(0.f);
    }
    __syncthreads();

    // ---- T = (I + diag(beta) Ab)^{-1}, blocked forward substitution
    if (w == 0) {
        const int base = lg * SUB, col = lr;
        float x[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
            float acc = (r == col) ? 1.f : 0.f;
            const float br = bet[base + r];
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= br * As[(base + r) * LA + base + i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < SUB; ++r) Ts[(base + r) * LA + base + col] = x[r];
    }
    __syncthreads();
    for (int R = 1; R < 4; ++R) {
        if (w < R) {
            const int I = w;
            f32x4 x = zero4();
            const float br = bet[R * SUB + lr];
            for (int J = I; J < R; ++J)
#pragma unroll
                for (int kk = 0; kk < SUB; kk += 4) {
                    const float a = br * As[(R * SUB + lr) * LA + J * SUB + kk + lg];
                    const float b = Ts[(J * SUB + kk + lg) * LA + I * SUB + lr];
                    x = mma4(a, b, x);
                }
            float* xs = Xs + I * SUB * SUB;
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[(4 * lg + e) * SUB + lr] = x[e];
            f32x4 y = zero4();
#pragma unroll
            for (int kk = 0; kk < SUB; kk += 4) {
                const float a = Ts[(R * SUB + lr) * LA + R * SUB + kk + lg];
                const float b = xs[(kk + lg) * SUB + lr];
                y = mma4(a, b, y);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Ts[(R * SUB + 4 * lg + e) * LA + I * SUB + lr] = -y[e];
        }
        __syncthreads();
    }

    // register fields of this wave's rows and column half
    f32x4 fQ[NCTH], fK[NCTH], fG[NCTH];
#pragma unroll
    for (int ct = 0; ct < NCTH; ++ct) fQ[ct] = fK[ct] = fG[ct] = zero4();
    auto qval = [&](int r, int c) -> float {
        if constexpr (L::QLDS) return to_f32(Qs[r * DKP + c]);
        return r < valid ? to_f32(q[(row0 + (size_t)r * H) * DK + c]) : 0.f;
    };
    auto vval = [&](int r, int j) -> float { return to_f32(Vs[r * DVP + j]); };
    auto kval = [&](int r, int c) -> float { return to_f32(Ks[r * DKP + c]); };
    // beta partial sums of this lane's 4 rows, reduced over the 16 lanes of a
    // row group; one array per column half (no two waves write one slot)
    auto add_dbeta = [&](f32x4 s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float t = s[e];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) t += __shfl_xor(t, off);
            if (lr == 0) dbt[hf * C + rowD + e] += t;
        }
    };

    // ---- dT = (dW Kg^T + dVn V^T) diag(beta), lower block pairs
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
        const int R = kPairsB[w][jp][0], I = kPairsB[w][jp][1];
        if (R < 0) break;
        const int ra = R * 16 + lr, ib = I * 16 + lr;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += 4) {
            const int c = kk + lg;
            acc = mma4(ob[OL::DWT + (size_t)c * C + ra], kval(ib, c) * dexp2<E>(Gs[ib * DKP + c]), acc);
        }
#pragma unroll
        for (int kk = 0; kk < DV; kk += 4) {
            const int j = kk + lg;
            acc = mma4(ob[OL::DVNT + (size_t)j * C + ra], vval(ib, j), acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = R * 16 + 4 * lg + e, i = I * 16 + lr;
            S1[r * LA + i] = i < r ? bet[i] * acc[e] : 0.f;
        }
    }
    for (int idx = tid; idx < 6 * SUB * SUB; idx += NTH) {
        int R, I;
        upper_block(idx / (SUB * SUB), R, I);
        const int e = idx % (SUB * SUB);
        S1[(R * SUB + e / SUB) * LA + I * SUB + e % SUB] = 0.f;
    }

    // ---- dBk = T^T dW (into dK, dG, dbeta) and dBv = T^T dVn (dV, dbeta):
    //      rows 16X.., this wave's column half
    {
        f32x4 sb = zero4();
#pragma unroll 1
        for (int ct = 0; ct < NCTH; ++ct) {
            const int c = (hf * NCTH + ct) * 16 + lr;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < C; kk += 4) {
                const int r = kk + lg;
                acc = mma4(Ts[r * LA + rowA], ob[OL::DWT + (size_t)c * C + r], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = rowD + e;
                const float gam = dexp2<E>(Gs[i * DKP + c]), kv = kval(i, c);
                const float bk = bet[i] * acc[e] * gam;          // (beta dBk) e^G
                sb[e] += acc[e] * kv * gam;                      // dBk . Kg
                fK[ct][e] += bk;
                fG[ct][e] += bk * kv;
            }
        }
#pragma unroll 1
        for (int jt = 0; jt < NVTH; ++jt) {
            const int j = (hf * NVTH + jt) * 16 + lr;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < C; kk += 4) {
                const int r = kk + lg;
                acc = mma4(Ts[r * LA + rowA], ob[OL::DVNT + (size_t)j * C + r], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = rowD + e;
                sb[e] += acc[e] * vval(i, j);
                if (i < valid) dvo[(row0 + (size_t)i * H) * DV + j] = bet[i] * acc[e];
            }
        }
        add_dbeta(sb);
    }
    __syncthreads();

    // ---- dA = tril_-1(-T^T dT T^T): S2 = dT T^T, then rows 16X.. of dA
    for (int it = 2 * hf; it < 2 * hf + 2; ++it) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < C; kk += 4) {
            const int b = kk + lg;
            acc = mma4(S1[rowA * LA + b], Ts[(it * 16 + lr) * LA + b], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) S2[(rowD + e) * LA + it * 16 + lr] = acc[e];
    }
    __syncthreads();
    {
        f32x4 sb = zero4();
        f32x4 dA[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int it = 2 * hf + u;
            f32x4 acc = zero4();
            if (it <= X) {
#pragma unroll
                for (int kk = 0; kk < C; kk += 4) {
                    const int a = kk + lg;
                    acc = mma4(Ts[a * LA + rowA], S2[a * LA + it * 16 + lr], acc);
                }
            }
            const int i = it * 16 + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rowD + e;
                const float d = i < r ? -acc[e] : 0.f;
                sb[e] += d * As[r * LA + i];
                acc[e] = bet[r] * d;
            }
            dA[u] = acc;
        }
        add_dbeta(sb);
        __syncthreads();   // S1 (dT) and S2 (dT T^T) are read by every wave above
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) S1[(rowD + e) * LA + (2 * hf + u) * 16 + lr] = dA[u][e];
        // dM (lower triangle, from the reverse chain) into S2
        for (int idx = tid; idx < C * C; idx += NTH) {
            const int i = idx / C, r = idx % C;
            S2[r * LA + i] = ob[OL::DMT + idx];
        }
        if constexpr (L::QLDS) {   // q over Ab (zero past the end)
            for (int idx = tid; idx < C * DK / 2; idx += NTH) {
                const int r = idx / (DK / 2), c = 2 * (idx % (DK / 2));
                const typename Pair<E>::type qq = load2<E>(q + (row0 + (size_t)min(r, last) * H) * DK + c);
                Qs[r * DKP + c] = r < valid ? qq[0] : from_f32<E>(0.f);
                Qs[r * DKP + c + 1] = r < valid ? qq[1] : from_f32<E>(0.f);
            }
        }
    }
    __syncthreads();

    // ---- decayed products: rows r of block X against blocks Y <= X,
    //   (beta dA) Kt and dM Kt (row side), and columns i of block X against
    //   blocks Y >= X: (beta dA)^T Kg and dM^T Qg (column side)
#pragma unroll 1
    for (int ct = 0; ct < NCTH; ++ct) {
        const int c = (hf * NCTH + ct) * 16 + lr;   // B-operand column = accumulator column of this lane
        f32x4 accA = zero4(), accC = zero4(), accB = zero4(), accD = zero4();
        for (int Y = 0; Y <= X; ++Y) {
            const float s = Y < X ? dsc[pair_index(X, Y) * DK + c] : 1.f;
            const float gY = gm[Y * DK + c];
#pragma unroll
            for (int ks = 0; ks < SUB; ks += 4) {
                const int y = Y * 16 + ks + lg;
                const float bkr = ((kval(y, c) * dexp2<E>(gY - Gs[y * DKP + c])) * s) * s;
                accA = mma4(S1[rowA * LA + y], bkr, accA);
                accC = mma4(S2[rowA * LA + y], bkr, accC);
            }
        }
        for (int Y = X; Y < 4; ++Y) {
            const float s = Y > X ? dsc[pair_index(Y, X) * DK + c] : 1.f;
            const float gY = gm[Y * DK + c];
#pragma unroll
            for (int ks = 0; ks < SUB; ks += 4) {
                const int y = Y * 16 + ks + lg;
                const float el = (dexp2<E>(Gs[y * DKP + c] - gY) * s) * s;
                accB = mma4(S1[y * LA + rowA], kval(y, c) * el, accB);
                accD = mma4(S2[y * LA + rowA], qval(y, c) * el, accD);
            }
        }
        const float gX = gm[X * DK + c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowD + e;
            const float gr = Gs[r * DKP + c];
            const float fr = dexp2<E>(gr - gX), fc = dexp2<E>(gX - gr);
            const float kv = kval(r, c), qv = qval(r, c);
            const float a = accA[e] * fr, cq = accC[e] * fr, bt = (accB[e] + accD[e]) * fc;
            fK[ct][e] += a + bt;
            fQ[ct][e] += cq;
            fG[ct][e] += a * kv + cq * qv - bt * kv;
        }
    }

    // ---- terms from the reverse chain: dQg e^G, dKc e^{G_C - G}, and the
    //      column sums of dKc e^{G_C - G} k for the last row's dG
#pragma unroll 1
    for (int ct = 0; ct < NCTH; ++ct) {
        const int c = (hf * NCTH + ct) * 16 + lr;
        const f32x4 dqg = *reinterpret_cast<const f32x4*>(ob + OL::DQGT + (size_t)c * C + rowD);
        const f32x4 dkc = *reinterpret_cast<const f32x4*>(ob + OL::DKCT + (size_t)c * C + rowD);
        float cs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowD + e;
            const float g = Gs[r * DKP + c];
            const float gam = dexp2<E>(g), ec = dexp2<E>(gm[4 * DK + c] - g);
            const float kv = kval(r, c), qv = qval(r, c);
            fQ[ct][e] += dqg[e] * gam;
            fK[ct][e] += dkc[e] * ec;
            const float t = dkc[e] * ec * kv;
            fG[ct][e] += dqg[e] * gam * qv - t;
            cs += t;
        }
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        if (lg == 0) car[w * DK + c] = cs;    // wave w covers only its half's columns
    }
    __syncthreads();
    if (X == 3 && lg == 3) {
#pragma unroll
        for (int ct = 0; ct < NCTH; ++ct) {
            const int c = (hf * NCTH + ct) * 16 + lr;
            fG[ct][3] += ob[OL::DGC + c] + car[(4 * hf) * DK + c] + car[(4 * hf + 1) * DK + c] +
                         car[(4 * hf + 2) * DK + c] + car[(4 * hf + 3) * DK + c];
        }
    }
    // outputs dq, dk; dG into LDS (G is no longer read)
#pragma unroll
    for (int ct = 0; ct < NCTH; ++ct) {
        const int c = (hf * NCTH + ct) * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rowD + e;
            if (r < valid) {
                dq[(row0 + (size_t)r * H) * DK + c] = fQ[ct][e];
                dk[(row0 + (size_t)r * H) * DK + c] = fK[ct][e];
            }
        }
    }
    __syncthreads();   // every read of G and of the column sums is done
#pragma unroll
    for (int ct = 0; ct < NCTH; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) Gs[(rowD + e) * DKP + (hf * NCTH + ct) * 16 + lr] = fG[ct][e];
    __syncthreads();

    // ---- dg = reverse cumulative sum of dG over the chunk, dz
    {
        const int c0 = 2 * (tid % L::CP), part = tid / L::CP, r0 = part * RP;
        float suf[RP][2];
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = RP - 1; i >= 0; --i) {
            s0 += Gs[(r0 + i) * DKP + c0];
            s1 += Gs[(r0 + i) * DKP + c0 + 1];
            suf[i][0] = s0;
            suf[i][1] = s1;
        }
        car[part * DK + c0] = s0;
        car[part * DK + c0 + 1] = s1;
        __syncthreads();
        float cr[2] = {0.f, 0.f};
#pragma unroll
        for (int p = 0; p < L::NPART; ++p)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (p > part) cr[j] += car[p * DK + c0 + j];
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
            if (r < valid) {
                const size_t off = (row0 + (size_t)r * H) * DK + c0;
                const typename Pair<E>::type zz = load2<E>(z + off);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float sg = 1.0f / (1.0f + expf(-to_f32(zz[j])));
                    dz[off + j] = (suf[i][j] + cr[j]) * g_min * sg * (1.0f - sg);
                }
            }
        }
    }
    if (tid < valid) dbeta[row0 + (size_t)tid * H] = dbt[tid] + dbt[C + tid];
}

// ---------------------------------------------------------------------------
// Per-chunk gradients, bf16 tokens: 512 threads on bf16 MFMA.  Wave w owns the
// token block X = w % 4 and the channel half w / 4 of dQ, dK and dG, held in
// registers in the (channel, token) orientation of the accumulators: rows
// cb + 4(l/16) + e of a 16-channel tile, column (token) 16X + l%16, so that
// each lane reads and writes four consecutive channels of one token.
// The decayed products use three operand families, each built once per chunk
// with one exponential per element and stored channel-major (token index
// contiguous): Kr = k e^{G_m(Y) - G}, Kc = k e^{G - G_m(Y)} and
// Qc = q e^{G - G_m(Y)}, Y the token's own 16-row block, so every factor lies
// within e^{+-8|g_min|}.  A product over the token blocks Y accumulates block
// by block, the accumulator scaled between blocks by the ratio of consecutive
// reference factors e^{G_m(Y) - G_m(Y-1)} <= 1 (Horner's scheme).
// dA comes from NP = -tril_-1(dVn Vn^T) (written by the reverse chain):
// dT T^T = dVn Vn^T (I + A)^T T^T = dVn Vn^T, and tril_-1(T^T X T^T) only
// reads the strictly lower part of X, so dA = tril_-1(-T^T dT T^T) =
// tril_-1(T^T NP).
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct DIntraH {
    static constexpr int NTH = 512, NW = 8;
    static constexpr int CP = DK / 2, NPART = NTH / CP, RP = C / NPART;   // gate scan: channel pairs x row parts
    static constexpr int NCTH = DK / 32, NVTH = DV / 32;                  // 16-wide tiles per half
    static constexpr int DKP = DK + 4, LY = C + 8, LT = C + 8;
    static constexpr int NCAR = NPART > 4 ? NPART : 4;
    static constexpr size_t OFF_G = 0;                                   // [C][DKP] fp32 G (log2), then dG
    static constexpr size_t OFF_KR = OFF_G + (size_t)C * DKP * 4;        // [DK][LY] bf16 Kr^T
    static constexpr size_t OFF_KC = OFF_KR + (size_t)DK * LY * 2;       // [DK][LY] bf16 Kc^T
    static constexpr size_t OFF_QC = OFF_KC + (size_t)DK * LY * 2;       // [DK][LY] bf16 Qc^T
    static constexpr size_t OFF_TT = OFF_QC + (size_t)DK * LY * 2;       // [C][C] bf16 T^T (swizzled)
    static constexpr size_t OFF_AB = OFF_TT + (size_t)C * C * 2;         // [C][C] bf16 Ab (swizzled)
    static constexpr size_t OFF_DA = OFF_AB + (size_t)C * C * 2;         // [C][LT] bf16 beta dA
    static constexpr size_t OFF_DAT = OFF_DA + (size_t)C * LT * 2;       // [C][LT] bf16 (beta dA)^T
    static constexpr size_t OFF_GM = OFF_DAT + (size_t)C * LT * 2;       // [5][DK] G_m(0..3), G_C
    static constexpr size_t OFF_RHO = OFF_GM + 5 * DK * 4;               // [3][DK] e^{G_m(Y+1) - G_m(Y)}
    static constexpr size_t OFF_CAR = OFF_RHO + 3 * DK * 4;              // [NCAR][DK]
    static constexpr size_t OFF_BET = OFF_CAR + (size_t)NCAR * DK * 4;   // [C]
    static constexpr size_t OFF_DB = OFF_BET + C * 4;                    // [6][C] dbeta partials
    static constexpr size_t LDS = OFF_DB + 6 * C * 4;
    static_assert(LDS <= 160 * 1024, "per-chunk gradient LDS budget");
    static_assert(RP % 2 == 0 && 16 % RP == 0 && DK % 32 == 0 && DV % 32 == 0, "tiling");
    static_assert(NCTH % 2 == 0 && NVTH % 2 == 0, "result tiles are stored in pairs");
    static_assert(2 * C * C * 2 == 2 * 1024 * NW, "T^T and Ab: two 1 KB loads per wave");
};

// T^T and Ab (64 x 64 bf16 each) into LDS by asynchronous global->LDS loads,
// two 1 KB wave instructions per wave of an 8-wave workgroup; group g (8
// elements) of row r lands at position g ^ (r mod 8) of its 128-byte row.
__device__ __forceinline__ void stage_tt_ab(const bf16* __restrict__ tt, const bf16* __restrict__ ab,
                                            unsigned char* lds_tt, unsigned char* lds_ab) {
    const int w = wave_id(), l = lane_id();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ins = w * 2 + i, mat = ins >> 3, byte = (ins & 7) * 1024 + 16 * l;
        const int r = byte / (C * 2), g = ((byte % (C * 2)) / 16) ^ (r & 7);
        __builtin_amdgcn_global_load_lds((mat ? ab : tt) + r * C + g * 8, (mat ? lds_ab : lds_tt) + (ins & 7) * 1024,
                                         16, 0, 0);
    }
}

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int DK, int DV>
__global__ __launch_bounds__(512) void dintra16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                       const bf16* __restrict__ v, const bf16* __restrict__ z,
                                                       const bf16* __restrict__ beta, float g_min, int T, int H,
                                                       int NC, const unsigned char* __restrict__ obuf,
                                                       const unsigned char* __restrict__ bws,
                                                       float* __restrict__ dq, float* __restrict__ dk,
                                                       float* __restrict__ dvo, float* __restrict__ dz,
                                                       float* __restrict__ dbeta) {
    typedef DIntraH<DK, DV> L;
    typedef ObH<DK, DV> OH;
    typedef Mfma<bf16> MF;
    constexpr int NTH = L::NTH, RP = L::RP, DKP = L::DKP, LY = L::LY, LT = L::LT;
    constexpr int NCTH = L::NCTH, NVTH = L::NVTH;
    constexpr float LOG2E = 1.4426950408889634f;
    extern __shared__ __align__(16) unsigned char smem[];
    float* Gs = reinterpret_cast<float*>(smem + L::OFF_G);
    bf16* KRt = reinterpret_cast<bf16*>(smem + L::OFF_KR);
    bf16* KCt = reinterpret_cast<bf16*>(smem + L::OFF_KC);
    bf16* QCt = reinterpret_cast<bf16*>(smem + L::OFF_QC);
    const bf16* TT = reinterpret_cast<const bf16*>(smem + L::OFF_TT);
    const bf16* AB = reinterpret_cast<const bf16*>(smem + L::OFF_AB);
    bf16* DA = reinterpret_cast<bf16*>(smem + L::OFF_DA);
    bf16* DAT = reinterpret_cast<bf16*>(smem + L::OFF_DAT);
    float* gm = reinterpret_cast<float*>(smem + L::OFF_GM);
    float* rho = reinterpret_cast<float*>(smem + L::OFF_RHO);
    float* car = reinterpret_cast<float*>(smem + L::OFF_CAR);
    float* bet = reinterpret_cast<float*>(smem + L::OFF_BET);
    float* dbp = reinterpret_cast<float*>(smem + L::OFF_DB);

    const int n = blockIdx.x, hh = blockIdx.y, bb = blockIdx.z;
    const int valid = min(C, T - n * C), last = valid - 1;
    const size_t row0 = ((size_t)bb * T + (size_t)n * C) * H + hh;   // token row of chunk row 0
    const unsigned char* obc = obuf + (((size_t)bb * H + hh) * NC + n) * OH::BYTES;
    const bf16* ob = reinterpret_cast<const bf16*>(obc);
    const float* dgc = reinterpret_cast<const float*>(obc + OH::DGC_BYTE);
    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int lr = l & 15, lg = l >> 4;
    const int X = w & 3, hf = w >> 2;   // token block and channel half of this wave
    const int rX = X * 16 + lr;         // token (accumulator column) of this lane
    const bf16* wb = reinterpret_cast<const bf16*>(bws + (((size_t)bb * H + hh) * NC + n) * WsB<bf16, DK, DV>::BYTES);

    // T^T and Ab (written by the forward half's intra-chunk kernel) into LDS
    // by asynchronous loads: rows of 64 bf16 in 16-byte groups, group g of row
    // r at position g ^ (r mod 8); they land before the barrier that ends the
    // operand families
    stage_tt_ab(wb + WsB<bf16, DK, DV>::TT, wb + WsB<bf16, DK, DV>::AB, smem + L::OFF_TT, smem + L::OFF_AB);
    // fragment (rows row0 + l%16, token columns k0 + 8(l/16) ..) of T^T, and an element of Ab
    auto tt_frag = [&](int row0, int k0) -> MF::frag {
        const int r = row0 + lr, g = k0 / 8 + lg;
        return *reinterpret_cast<const MF::frag*>(TT + r * C + ((g ^ (r & 7)) << 3));
    };
    auto ab_elem = [&](int r, int i) -> float {
        return to_f32(AB[r * C + ((((i >> 3) ^ (r & 7)) << 3) | (i & 7))]);
    };
    // this wave's block pairs (R, I), and the reverse chain's operands of the
    // dA phase and the decayed products: NP^T of the pairs, dM and dM^T rows
    // of this lane's token (every block); issued here to be in flight during
    // the gate scan and the operand families
    const int I0 = kPairsB[w][0][1], I1 = kPairsB[w][1][1];
    const bool two = kPairsB[w][1][0] >= 0;
    bf16x8 npf[2][C / 32];
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
        npf[0][kb] = *reinterpret_cast<const bf16x8*>(ob + OH::NPT + tix(I0 * 16 + lr, kb * 32 + lg * 8, C));
        npf[1][kb] = two ? *reinterpret_cast<const bf16x8*>(ob + OH::NPT + tix(I1 * 16 + lr, kb * 32 + lg * 8, C))
                         : bf16x8{};
    }
    bf16x4 dmr[4], dmc[4];
#pragma unroll
    for (int Y = 0; Y < 4; ++Y) {
        dmr[Y] = *reinterpret_cast<const bf16x4*>(ob + OH::DM + tix(rX, Y * 16 + 4 * lg, C));
        dmc[Y] = *reinterpret_cast<const bf16x4*>(ob + OH::DMT + tix(rX, Y * 16 + 4 * lg, C));
    }

    // the operand families' token loads (two tokens x eight channels per
    // thread) are issued first, to be in flight during the gate scan
    constexpr int NFAM = (C / 2) * (DK / 8);
    static_assert(NFAM <= NTH, "one family item per thread");
    const bool fam = tid < NFAM;
    const int fy0 = 2 * (tid % (C / 2)), fc8 = (tid / (C / 2)) * 8 % DK;
    bf16x8 fk[2], fq[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const size_t off = (row0 + (size_t)min(fy0 + u, last) * H) * DK + fc8;
        fk[u] = *reinterpret_cast<const bf16x8*>(k + off);
        fq[u] = *reinterpret_cast<const bf16x8*>(q + off);
    }

    // ---- gate, chunk-local scan (log2 units)
    {
        const int c0 = 2 * (tid % L::CP), part = tid / L::CP, r0 = part * RP;
        const float kg2 = g_min * LOG2E;
        float G[RP][2];
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
            const bf16x2 zz = load2<bf16>(z + (row0 + (size_t)min(r, last) * H) * DK + c0);
            const bool ok = r < valid;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float g2 = kg2 * __builtin_amdgcn_rcpf(1.0f + dexp2<bf16>(-LOG2E * to_f32(zz[j])));
                G[i][j] = ok ? g2 : 0.f;
            }
            s0 += G[i][0];
            s1 += G[i][1];
            G[i][0] = s0;
            G[i][1] = s1;
        }
        car[part * DK + c0] = s0;
        car[part * DK + c0 + 1] = s1;
        if (tid < C) bet[tid] = tid < valid ? to_f32(beta[row0 + (size_t)tid * H]) : 0.f;
        for (int idx = tid; idx < 6 * C; idx += NTH) dbp[idx] = 0.f;
        __syncthreads();
        float cr[2] = {0.f, 0.f}, gC[2] = {0.f, 0.f};
#pragma unroll
        for (int p = 0; p < L::NPART; ++p)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float t = car[p * DK + c0 + j];
                if (p < part) cr[j] += t;
                gC[j] += t;
            }
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float g = G[i][j] + cr[j];
                Gs[r * DKP + c0 + j] = g;
                if ((r & 15) == 7) gm[(r >> 4) * DK + c0 + j] = g;
            }
        }
        if (part == 0) {
            gm[4 * DK + c0] = gC[0];
            gm[4 * DK + c0 + 1] = gC[1];
        }
        __syncthreads();
    }
    // reference ratios e^{G_m(Y+1) - G_m(Y)}
    for (int idx = tid; idx < 3 * DK; idx += NTH) {
        const int p = idx / DK, cc = idx % DK;
        rho[idx] = dexp2<bf16>(gm[(p + 1) * DK + cc] - gm[p * DK + cc]);
    }
    // operand families, channel-major
    if (fam) {
        const int Y = fy0 >> 4;
        float kr[2][8], kc[2][8], qc[2][8];
        const f32x4 ma = *reinterpret_cast<const f32x4*>(gm + Y * DK + fc8);
        const f32x4 mb = *reinterpret_cast<const f32x4*>(gm + Y * DK + fc8 + 4);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int y = fy0 + u;
            const bool ok = y < valid;
            const f32x4 ga = *reinterpret_cast<const f32x4*>(Gs + y * DKP + fc8);
            const f32x4 gb = *reinterpret_cast<const f32x4*>(Gs + y * DKP + fc8 + 4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float d = (j < 4 ? ma[j] : mb[j - 4]) - (j < 4 ? ga[j] : gb[j - 4]);
                const float e1 = dexp2<bf16>(d), e2 = dexp2<bf16>(-d);
                const float kv = ok ? to_f32(fk[u][j]) : 0.f, qv = ok ? to_f32(fq[u][j]) : 0.f;
                kr[u][j] = kv * e1;
                kc[u][j] = kv * e2;
                qc[u][j] = qv * e2;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            store2<bf16>(KRt + (fc8 + j) * LY + fy0, kr[0][j], kr[1][j]);
            store2<bf16>(KCt + (fc8 + j) * LY + fy0, kc[0][j], kc[1][j]);
            store2<bf16>(QCt + (fc8 + j) * LY + fy0, qc[0][j], qc[1][j]);
        }
    }
    const size_t trow = row0 + (size_t)min(rX, last) * H;   // token row of rX, clamped in bounds
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's T^T / Ab loads have landed
    __syncthreads();

    // ---- dA = tril_-1(T^T NP) per block pair, in both orientations; the
    //      dA . Ab part of dbeta, one partial slot per column block I
    f32x4 d1[2], d2[2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
        const int R = kPairsB[w][jp][0], I = kPairsB[w][jp][1];
        d1[jp] = d2[jp] = zero4();
        if (R < 0) continue;
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb) {
            const MF::frag ft = tt_frag(R * 16, kb * 32);
            d1[jp] = MF::mma(ft, npf[jp][kb], d1[jp]);   // (row r, column i)
            d2[jp] = MF::mma(npf[jp][kb], ft, d2[jp]);   // (row i, column r)
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = R * 16 + 4 * lg + e, i = I * 16 + lr;
            d1[jp][e] = i < r ? d1[jp][e] : 0.f;
            const float t = sum16(d1[jp][e] * ab_elem(r, i));
            if (lr == 0) dbp[I * C + r] = t;
            d2[jp][e] = (I * 16 + 4 * lg + e < R * 16 + lr) ? d2[jp][e] : 0.f;
        }
    }
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
        const int R = kPairsB[w][jp][0], I = kPairsB[w][jp][1];
        if (R < 0) continue;
        const int r = R * 16 + lr, i0 = I * 16 + 4 * lg;
        store4<bf16>(DA + r * LT + i0, d2[jp] * bet[r]);
        const int i = I * 16 + lr, r0 = R * 16 + 4 * lg;
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = d1[jp][e] * bet[r0 + e];
        store4<bf16>(DAT + i * LT + r0, t);
    }
    // exact zeros outside the triangles: the upper blocks of beta dA and the
    // lower blocks of its transpose
    for (int idx = tid; idx < 6 * SUB * SUB; idx += NTH) {
        int R, I;
        upper_block(idx / (SUB * SUB), R, I);   // I > R
        const int e = idx % (SUB * SUB);
        DA[(R * SUB + e / SUB) * LT + I * SUB + e % SUB] = from_f32<bf16>(0.f);
        DAT[(I * SUB + e / SUB) * LT + R * SUB + e % SUB] = from_f32<bf16>(0.f);
    }
    __syncthreads();

    // ---- per channel tile: dBk = T^T dW, the decayed products and the
    //      reverse chain's terms, into the register fields; each tile's
    //      global operands are loaded one tile ahead
    const float brX = bet[rX];
    const bool okX = rX < valid;
    struct Tile {
        bf16x8 w[C / 32];
        bf16x4 k4, q4, dqg, dkc;
    };
    auto load_tile = [&](int ct, Tile& t) {
        const int cb = hf * (DK / 2) + ct * 16, c4 = cb + 4 * lg;
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb)
            t.w[kb] = *reinterpret_cast<const bf16x8*>(ob + OH::DWT + tix(cb + lr, kb * 32 + lg * 8, C));
        t.k4 = load_raw4<bf16>(k + trow * DK + c4);
        t.q4 = load_raw4<bf16>(q + trow * DK + c4);
        t.dqg = load_raw4<bf16>(ob + OH::DQG + tix(rX, c4, DK));
        t.dkc = load_raw4<bf16>(ob + OH::DKC + tix(rX, c4, DK));
    };
    f32x4 fG[NCTH];   // dq and dk are final within their tile and stored there
    float sb = 0.f;   // dbeta partial of token rX
    bf16x8 dvf[NVTH][C / 32];   // dVn^T tiles of this wave's value half, and v
    bf16x4 vr[NVTH];
    // results of rows X*16 + (l >> 3) (+ 8), 16 bytes at channel 4 (l & 7) of a tile pair
    const int prow = X * 16 + (l >> 3), pj = 4 * (l & 7);
    auto put_pair = [&](float* dst, int ld, int c0, const f32x4& P, const f32x4& Q) {
        f32x4 lo, hi;
        pair_rows(P, Q, lo, hi);
        if (prow < valid) *reinterpret_cast<f32x4*>(dst + (row0 + (size_t)prow * H) * ld + c0 + pj) = lo;
        if (prow + 8 < valid) *reinterpret_cast<f32x4*>(dst + (row0 + (size_t)(prow + 8) * H) * ld + c0 + pj) = hi;
    };
    f32x4 pQ, pK;   // the even tile of a pair, stored with the odd one
    auto tile_step = [&](const int ct, const Tile& cur) {
        const int cb = hf * (DK / 2) + ct * 16, c4 = cb + 4 * lg;
        f32x4 accK = zero4();
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb) accK = MF::mma(cur.w[kb], tt_frag(X * 16, kb * 32), accK);
        // the token blocks Y accumulate by Horner's scheme, branch-free: the
        // accumulator is scaled by e^{G_m(Y) - G_m(Y-1)} (row side, upward) or
        // e^{G_m(Y+1) - G_m(Y)} (column side, downward) inside the triangle and
        // by 1 outside it, where the products add exact zeros (upper blocks of
        // beta dA and dM); the selects are on the wave-uniform X
        const f32x4 one4 = f32x4{1.f, 1.f, 1.f, 1.f};
        f32x4 accA = zero4(), accC = zero4();
#pragma unroll
        for (int Y = 0; Y < 4; ++Y) {
            const int fo = (cb + lr) * LY + Y * 16 + 4 * lg, ao = rX * LT + Y * 16 + 4 * lg;
            const bf16x4 fa = *reinterpret_cast<const bf16x4*>(KRt + fo);
            if (Y > 0) {
                const f32x4 rr = *reinterpret_cast<const f32x4*>(rho + (Y - 1) * DK + c4);
                const f32x4 sc = Y <= X ? rr : one4;
                accA *= sc;
                accC *= sc;
            }
            accA = mma16(fa, *reinterpret_cast<const bf16x4*>(DA + ao), accA);
            accC = mma16(fa, dmr[Y], accC);
        }
        f32x4 accB = zero4(), accD = zero4();
#pragma unroll
        for (int Y = 3; Y >= 0; --Y) {
            const int fo = (cb + lr) * LY + Y * 16 + 4 * lg, ao = rX * LT + Y * 16 + 4 * lg;
            const bf16x4 fk = *reinterpret_cast<const bf16x4*>(KCt + fo);
            const bf16x4 fq = *reinterpret_cast<const bf16x4*>(QCt + fo);
            if (Y < 3) {
                const f32x4 rr = *reinterpret_cast<const f32x4*>(rho + Y * DK + c4);
                const f32x4 sc = Y >= X ? rr : one4;
                accB *= sc;
                accD *= sc;
            }
            accB = mma16(fk, *reinterpret_cast<const bf16x4*>(DAT + ao), accB);
            accD = mma16(fq, dmc[Y], accD);
        }
        const f32x4 G4 = *reinterpret_cast<const f32x4*>(Gs + rX * DKP + c4);
        const f32x4 gX = *reinterpret_cast<const f32x4*>(gm + X * DK + c4);
        const f32x4 gC = *reinterpret_cast<const f32x4*>(gm + 4 * DK + c4);
        const f32x4 k4 = okX ? widen4(cur.k4) : zero4();
        const f32x4 q4 = okX ? widen4(cur.q4) : zero4();
        const f32x4 dqg = widen4(cur.dqg), dkc = widen4(cur.dkc);
        f32x4 cs, fQ, fK;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float gam = dexp2<bf16>(G4[e]), ec = dexp2<bf16>(gC[e] - G4[e]);
            const float fr = dexp2<bf16>(G4[e] - gX[e]), fc = dexp2<bf16>(gX[e] - G4[e]);
            const float bk = brX * accK[e] * gam;               // beta dBk e^G
            sb += accK[e] * k4[e] * gam;                        // dBk . Kg
            const float a = accA[e] * fr, cq = accC[e] * fr, bt = (accB[e] + accD[e]) * fc;
            const float t = dkc[e] * ec * k4[e];
            fQ[e] = cq + dqg[e] * gam;
            fK[e] = bk + a + bt + dkc[e] * ec;
            // the decayed products' dG terms take their k and q factors from the
            // same rounded families as the MFMA operands (k_r e^{G_r - G_m(X)} is
            // Kc of row r, and so on): the row-side and column-side terms then
            // cancel in the chunk's sum of dG as they do exactly
            const int co = (c4 + e) * LY + rX;
            fG[ct][e] = bk * k4[e] + accA[e] * to_f32(KCt[co]) + accC[e] * to_f32(QCt[co]) -
                        (accB[e] + accD[e]) * to_f32(KRt[co]) + dqg[e] * gam * q4[e] - t;
            cs[e] = t;
        }
        // column sums of dKc e^{G_C - G} k over this wave's 16 tokens
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[e] = sum16(cs[e]);
        if (lr == 0) *reinterpret_cast<f32x4*>(car + X * DK + c4) = cs;
        if (ct & 1) {
            put_pair(dq, DK, cb - 16, pQ, fQ);
            put_pair(dk, DK, cb - 16, pK, fK);
        } else {
            pQ = fQ;
            pK = fK;
        }
    };
    // straight-line prefetch (no branch in the loop, so the waits before
    // a tile's first use count only the loads issued after its own)
    Tile cur;
    load_tile(0, cur);
#pragma unroll 1
    for (int ct = 0; ct < NCTH - 1; ++ct) {
        Tile nxt;
        load_tile(ct + 1, nxt);
        tile_step(ct, cur);
        cur = nxt;
    }
    // the last tile, with the dBv operands loaded ahead
#pragma unroll
    for (int jt = 0; jt < NVTH; ++jt) {
        const int jb = hf * (DV / 2) + jt * 16;
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb)
            dvf[jt][kb] = *reinterpret_cast<const bf16x8*>(ob + OH::DVNT + tix(jb + lr, kb * 32 + lg * 8, C));
        vr[jt] = load_raw4<bf16>(v + trow * DV + jb + 4 * lg);
    }
    tile_step(NCTH - 1, cur);
    // ---- dBv = T^T dVn: dV and the dBv . V part of dbeta
    f32x4 pV;
#pragma unroll
    for (int jt = 0; jt < NVTH; ++jt) {
        const int jb = hf * (DV / 2) + jt * 16, j4 = jb + 4 * lg;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb) acc = MF::mma(dvf[jt][kb], tt_frag(X * 16, kb * 32), acc);
        const f32x4 v4 = okX ? widen4(vr[jt]) : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) sb += acc[e] * v4[e];
        if (jt & 1)
            put_pair(dvo, DV, jb - 16, pV, acc * brX);
        else
            pV = acc * brX;
    }
    sb += __shfl_xor(sb, 16);
    sb += __shfl_xor(sb, 32);
    if (lg == 0) dbp[(4 + hf) * C + rX] = sb;
    __syncthreads();   // column sums complete
    if (X == 3 && lr == 15) {   // the chunk's last row carries the G_C terms
#pragma unroll
        for (int ct = 0; ct < NCTH; ++ct) {
            const int c4 = hf * (DK / 2) + ct * 16 + 4 * lg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = c4 + e;
                fG[ct][e] += dgc[c] + car[c] + car[DK + c] + car[2 * DK + c] + car[3 * DK + c];
            }
        }
    }
    __syncthreads();   // every read of G and of the column sums is done
#pragma unroll
    for (int ct = 0; ct < NCTH; ++ct)
        *reinterpret_cast<f32x4*>(Gs + rX * DKP + hf * (DK / 2) + ct * 16 + 4 * lg) = fG[ct];
    __syncthreads();

    // ---- dg = reverse cumulative sum of dG over the chunk, dz
    {
        // z is read again here; an opaque copy of the pointer keeps the
        // compiler from holding the gate scan's loads in registers until now
        const bf16* zl = z;
        asm volatile("" : "+s"(zl));
        const int c0 = 2 * (tid % L::CP), part = tid / L::CP, r0 = part * RP;
        // this thread's logits, issued before the sums they wait for
        bf16x2 zz[RP];
#pragma unroll
        for (int i = 0; i < RP; ++i)
            zz[i] = load2<bf16>(zl + (row0 + (size_t)min(r0 + i, valid - 1) * H) * DK + c0);
        float suf[RP][2];
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = RP - 1; i >= 0; --i) {
            s0 += Gs[(r0 + i) * DKP + c0];
            s1 += Gs[(r0 + i) * DKP + c0 + 1];
            suf[i][0] = s0;
            suf[i][1] = s1;
        }
        car[part * DK + c0] = s0;
        car[part * DK + c0 + 1] = s1;
        __syncthreads();
        float cr[2] = {0.f, 0.f};
#pragma unroll
        for (int p = 0; p < L::NPART; ++p)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (p > part) cr[j] += car[p * DK + c0 + j];
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            const int r = r0 + i;
            if (r < valid) {
                const size_t off = (row0 + (size_t)r * H) * DK + c0;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float sg = __builtin_amdgcn_rcpf(1.0f + dexp2<bf16>(-LOG2E * to_f32(zz[i][j])));
                    dz[off + j] = (suf[i][j] + cr[j]) * g_min * sg * (1.0f - sg);
                }
            }
        }
    }
    if (tid < valid)
        dbeta[row0 + (size_t)tid * H] = dbp[tid] + dbp[C + tid] + dbp[2 * C + tid] + dbp[3 * C + tid] +
                                        dbp[4 * C + tid] + dbp[5 * C + tid];
}

template <class E, int DK, int DV>
hipError_t launch_t(const BwdArgs& a) {
    typedef typename Compute<E>::type CT;
    const Lay lo = lay_t<CT, DK, DV>(a.B, a.T, a.H);
    unsigned char* ws = (unsigned char*)a.workspace;
    hipStream_t st = (hipStream_t)a.stream;
    const int NC = (a.T + C - 1) / C;
    hipError_t err = launch_chunk_bwd_forward(a, ws + lo.fws, ws + lo.bws, ws + lo.st, ws + lo.vn);
    if (err != hipSuccess) return err;
    typedef DChain<E, DK, DV> LC_;
    if ((err = hipFuncSetAttribute((const void*)dchain_kernel<E, DK, DV>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)LC_::LDS)) != hipSuccess)
        return err;
    hipLaunchKernelGGL((dchain_kernel<E, DK, DV>), dim3(a.B * a.H), dim3(LC_::NTH), LC_::LDS, st, (const E*)a.dout,
                       a.ds_final, a.ds0, a.T, a.H, NC, (const unsigned char*)(ws + lo.fws),
                       (const unsigned char*)(ws + lo.bws), (const CT*)(ws + lo.st), (const CT*)(ws + lo.vn),
                       ws + lo.ob);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if constexpr (std::is_same<E, bf16>::value) {
        typedef DIntraH<DK, DV> LI;
        if ((err = hipFuncSetAttribute((const void*)dintra16_kernel<DK, DV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LI::LDS)) != hipSuccess)
            return err;
        hipLaunchKernelGGL((dintra16_kernel<DK, DV>), dim3(NC, a.H, a.B), dim3(LI::NTH), LI::LDS, st,
                           (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.z,
                           (const bf16*)a.beta, a.g_min, a.T, a.H, NC, (const unsigned char*)(ws + lo.ob),
                           (const unsigned char*)(ws + lo.bws), a.dq, a.dk, a.dv, a.dz, a.dbeta);
    } else {
        typedef DIntra<E, DK, DV> LI;
        if ((err = hipFuncSetAttribute((const void*)dintra_kernel<E, DK, DV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LI::LDS)) != hipSuccess)
            return err;
        hipLaunchKernelGGL((dintra_kernel<E, DK, DV>), dim3(NC, a.H, a.B), dim3(LI::NTH), LI::LDS, st, (const E*)a.q,
                           (const E*)a.k, (const E*)a.v, (const E*)a.z, (const E*)a.beta, a.g_min, a.T, a.H, NC,
                           (const unsigned char*)(ws + lo.ob), a.dq, a.dk, a.dv, a.dz, a.dbeta);
    }
    return hipGetLastError();
}

// fp32 tokens: the reverse chain's LDS holds fp32 tiles, which fit for d_v = 64
bool chunkwise(int dk, int dv, bool bf16) { return bf16 || dv == 64; }

template <class CT>
size_t ws_t(int B, int T, int H, int dk, int dv) {
    if (dk == 128 && dv == 128) return lay_t<CT, 128, 128>(B, T, H).total;
    if (dk == 128 && dv == 64) return lay_t<CT, 128, 64>(B, T, H).total;
    if (dk == 64 && dv == 128) return lay_t<CT, 64, 128>(B, T, H).total;
    return lay_t<CT, 64, 64>(B, T, H).total;
}

hipError_t launch_bf16(const BwdArgs& a) {
    if (a.dk_dim == 128 && a.dv_dim == 128) return launch_t<bf16, 128, 128>(a);
    if (a.dk_dim == 128 && a.dv_dim == 64) return launch_t<bf16, 128, 64>(a);
    if (a.dk_dim == 64 && a.dv_dim == 128) return launch_t<bf16, 64, 128>(a);
    return launch_t<bf16, 64, 64>(a);
}

hipError_t launch_f32(const BwdArgs& a) {   // d_v = 64 only (chunkwise())
    if (a.dk_dim == 128) return launch_t<float, 128, 64>(a);
    return launch_t<float, 64, 64>(a);
}

}  // namespace bwdc

size_t chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, bool half) {
    const size_t seq = bwd_workspace_bytes(B, T, H, dk, dv);
    if (!bwdc::chunkwise(dk, dv, half)) return seq;
    const size_t ch = half ? bwdc::ws_t<bf16>(B, T, H, dk, dv)
                           : (dk == 128 ? bwdc::lay_t<float, 128, 64>(B, T, H).total
                                        : bwdc::lay_t<float, 64, 64>(B, T, H).total);
    return ch > seq ? ch : seq;
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
    if (a.T == 0 || a.g_min < CHUNK_G_MIN_LIMIT || !bwdc::chunkwise(a.dk_dim, a.dv_dim, a.bf16)) return launch_bwd(a);
    return a.bf16 ? bwdc::launch_bf16(a) : bwdc::launch_f32(a);
}

}  // namespace kda
