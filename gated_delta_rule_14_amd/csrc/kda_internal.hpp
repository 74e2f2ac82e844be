// kda_internal.hpp -- launcher interface between the host entry points
// (kda_api.hip) and the kernel translation units.  Arguments have already
// been validated when a launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

struct DecodeArgs {
    const void *q, *k, *v, *z, *beta;
    float g_min;
    float* state;
    void* o;               // raw read-out, or NULL
    int B, H, dk, dv;
    bool bf16;
    void* stream;
    // fused epilogue (gate != NULL): y = RMSNorm(o) * sigmoid(gate), written
    // to y in the token dtype, or as bf16 when y_bf16 is set
    const void* gate = nullptr;
    float eps = 0.f;
    void* y = nullptr;
    bool y_bf16 = false;
    // z holds one logit per (b, h) for all d_k channels (scalar decay)
    bool z_scalar = false;
};
hipError_t launch_decode(const DecodeArgs& a);

// The DPLR recurrence: the whole sequence (step false) or one token on a
// state held in HBM (step true: s_final is that state, T unused).
struct DplrArgs {
    const void *q, *k, *v, *z, *a, *b;
    float g_min;
    const float* s0;
    void* o;
    float* s_final;
    int B, T, H, dk, dv;
    bool bf16, step;
    void* stream;
};
hipError_t launch_dplr(const DplrArgs& x);
// chunkwise DPLR prefill (dplr_chunk.hip); the workspace holds
// dplr_chunk_workspace_bytes() bytes
size_t dplr_chunk_workspace_bytes(int B, int T, int H, int dk, int dv, bool bf16);
hipError_t launch_dplr_chunk(const DplrArgs& x, void* workspace);
// zfull (rows x dk) = each of the rows scalar logits zs repeated dk times
hipError_t launch_broadcast_gate(const void* zs, void* zfull, size_t rows, int dk, bool bf16, void* stream);

// The chunkwise kernels' decay factors are bounded (finite, with negligible
// underflow) for g_min >= CHUNK_G_MIN_LIMIT; below it the prefill calls run
// the token-sequential kernel (seq.hip), exact for any g_min < 0.
constexpr float CHUNK_G_MIN_LIMIT = -8.0f;

struct ChunkArgs {
    const void *q, *k, *v, *z, *beta;
    float g_min;
    const float* s0;
    void* o;
    float* s_final;
    int B, T, H, dk, dv;
    bool bf16;
    void* workspace;
    void* stream;
    // fused output epilogue (gate != NULL; only where chunk_gate_fused()):
    // y = RMSNorm(o) * sigmoid(gate), laid out like o; o may then be NULL
    const void* gate = nullptr;
    float eps = 0.f;
    void* y = nullptr;
    // z holds one logit per (token, head), shape (B, T, H): the scalar gate,
    // read directly by the pipelined kernels (only where
    // chunk_scalar_gate_native())
    bool scalar_z = false;
};
size_t chunk_workspace_bytes(int B, int T, int H, int dk, int dv, bool bf16);
// whether the prefill kernels for these sizes run the output epilogue in
// their own launches (bf16 tokens, d_k = d_v = 128, the pipelined kernels on
// a segmented plan, whose light expand has LDS to stage the outputs)
bool chunk_gate_fused(int B, int T, int H, int dk, int dv, bool bf16);
// whether the prefill kernels for these sizes read a scalar gate directly
// (bf16 tokens, d_k = d_v = 128, the pipelined kernels, chunkwise g_min)
bool chunk_scalar_gate_native(int T, int dk, int dv, bool bf16, float g_min);
hipError_t launch_chunk(const ChunkArgs& a);
// token-sequential prefill (any g_min; with gate != NULL also the epilogue,
// y in the token dtype)
hipError_t launch_seq(const ChunkArgs& a);
// bf16 tokens: fused segment kernels (seg.hip); fp32 tokens: per-chunk
// workspace kernels (chunk.hip).  Both use the segment scan of chunk.hip.
size_t seg_workspace_bytes(int B, int T, int H, int dk, int dv);
hipError_t launch_chunk_seg(const ChunkArgs& a);
hipError_t launch_seg_scan(const float* P, const float* R, const float* s0, float* Sent, float* s_final, int nseg,
                           int nchain, int dk, int dv, void* stream);

struct GateArgs {
    const void *o, *gate;
    float eps;
    const void* w;
    void* y;
    int B, T, H, dv, d_model;
    bool bf16;
    void* workspace;
    void* stream;
};
size_t gate_workspace_bytes(int B, int T, int H, int dv, int d_model, bool bf16, bool proj);
hipError_t launch_out_gate(const GateArgs& a);
// The epilogue (bf16, d_v = 128) on tokens [0, t_a) and [t_b, T) of each
// sequence, o -> y (o may be y): the rows the split prefill plan's full
// expands leave to it.
hipError_t launch_gate_ends(const void* o, const void* gate, float eps, void* y, int B, int T, int H, int t_a, int t_b,
                            void* stream);
// out (M x N, bf16) = y (M x K, bf16) . w (N x K, bf16)^T (gemm.hip); N a
// multiple of 16, K of 64; scratch holds projection_scratch_bytes(M, N, K)
// bytes (fp32 partial tiles of a split K range for small M, else none)
size_t projection_scratch_bytes(int M, int N, int K);
bool gemm_small_m(int M);
hipError_t launch_projection(const void* y, const void* w, void* out, int M, int N, int K, void* scratch,
                             void* stream);

// Gradients of the recurrence (bwd.hip): token-sequential, one workgroup
// per (b, h); fp32 gradients.
struct BwdArgs {
    const void *q, *k, *v, *z, *beta;
    float g_min;
    const float* s0;
    const void* dout;
    const float* ds_final;
    float *dq, *dk, *dv, *dz, *dbeta, *ds0;
    int B, T, H, dk_dim, dv_dim;
    bool bf16;
    void* workspace;
    void* stream;
};
size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv);
hipError_t launch_bwd(const BwdArgs& a);

// Chunkwise gradients (kda_chunk_bwd): the forward half in chunk.hip (the
// per-chunk operands of both directions, then each chunk's entering state and
// V_new), the reverse chunk recurrence and the per-chunk gradients in
// bwd_chunk.hip.  g_min below CHUNK_G_MIN_LIMIT and T == 0 run launch_bwd.
hipError_t launch_chunk_bwd_forward(const BwdArgs& a, unsigned char* fws, unsigned char* bws, void* states,
                                    void* vn);
size_t chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, bool bf16);
hipError_t launch_chunk_bwd(const BwdArgs& a);

}  // namespace kda
