// kda_api.hip -- the C ABI of libkda (declared in include/kda.h): argument
// validation on the host, workspace sizing, and kernel dispatch.  Nothing
// here allocates device memory or synchronises, unless KDA_DEBUG_SYNC=1.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.hpp"

static_assert(kda::CHUNK_G_MIN_LIMIT == KDA_CHUNK_G_MIN_LIMIT, "one decay bound");

namespace {

bool debug_sync() {
    static int flag = -1;
    if (flag < 0) {
        const char* e = getenv("KDA_DEBUG_SYNC");
        flag = (e && e[0] == '1') ? 1 : 0;
    }
    return flag == 1;
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

bool dim_ok(int d) { return d == 64 || d == 128; }

kda_status finish(hipError_t err, void* stream) {
    if (err != hipSuccess) return KDA_ERR_HIP;
    if (debug_sync()) {
        if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KDA_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

// Checks shared by the prefill calls, in the order the header documents.
// KDA_OK with B * H == 0 means there is nothing to launch (pointers are not
// examined then).
kda_status check_chunk_args(const void* q, const void* k, const void* v, const void* z, const void* beta,
                            float g_min, const float* s0, const void* o, const float* s_final, int B, int T, int H,
                            int dk, int dv, int chunk, kda_dtype dt, const void* workspace) {
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_SHAPE;
    if (chunk != 64 || !dim_ok(dk) || !dim_ok(dv) || (dt != KDA_F32 && dt != KDA_BF16))
        return KDA_ERR_UNSUPPORTED;
    if (B > 65535 || H > 65535 || (long long)B * H * T > (1LL << 40)) return KDA_ERR_SHAPE;
    if (!(g_min < 0.f) || !isfinite(g_min)) return KDA_ERR_ARG;
    if (B == 0 || H == 0) return KDA_OK;
    if (T > 0 && (!q || !k || !v || !z || !beta || !o)) return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(z) || !aligned16(beta) ||
        !aligned16(s0) || !aligned16(o) || !aligned16(s_final) || !aligned16(workspace))
        return KDA_ERR_ALIGN;
    return KDA_OK;
}

// Checks shared by the decode calls (the state and token tensors of one step).
kda_status check_step_args(const void* q, const void* k, const void* v, const void* z, const void* beta,
                           float g_min, const float* state, int B, int H, int dk, int dv, kda_dtype dt) {
    if (B < 0 || H < 0) return KDA_ERR_SHAPE;
    if (!dim_ok(dk) || !dim_ok(dv) || (dt != KDA_F32 && dt != KDA_BF16)) return KDA_ERR_UNSUPPORTED;
    if ((long long)B * H > 0x7fffffffLL) return KDA_ERR_SHAPE;
    if (!(g_min < 0.f) || !isfinite(g_min)) return KDA_ERR_ARG;
    if (B == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !z || !beta || !state) return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(z) || !aligned16(beta) || !aligned16(state))
        return KDA_ERR_ALIGN;
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is negative or too large";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported d_k, d_v, chunk or dtype";
        case KDA_ERR_ARG: return "KDA_ERR_ARG: invalid scalar argument";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: pointer not 16-byte aligned";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP launch or execution error";
        case KDA_ERR_SCRATCH:
            return "KDA_ERR_SCRATCH: the call needs more scratch than kda_chunk_fwd_noalloc's static array holds";
    }
    return "KDA_ERR_?: unknown status";
}

const char* kda_version(void) { return "libkda 0.1 gfx950"; }

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, kda_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || chunk != 64 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    if (dt != KDA_F32 && dt != KDA_BF16) return 0;
    return kda::chunk_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16);
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* z, const void* beta,
                         float g_min, const float* s0, void* o, float* s_final, int B, int T, int H,
                         int dk, int dv, int chunk, kda_dtype dt, void* workspace, size_t workspace_bytes,
                         void* stream) {
    const kda_status st = check_chunk_args(q, k, v, z, beta, g_min, s0, o, s_final, B, T, H, dk, dv, chunk, dt,
                                           workspace);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    const size_t need = kda::chunk_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    kda::ChunkArgs a{q, k, v, z, beta, g_min, s0, o, s_final, B, T, H, dk, dv, dt == KDA_BF16,
                     workspace, stream};
    return finish(kda::launch_chunk(a), stream);
}

}  // extern "C"

namespace {

// The scratch of kda_chunk_fwd_noalloc.  In host code `scratch` names a
// host-side stand-in, not the device array: its device address, one per GPU
// (each GPU holds its own copy), comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is passed on.
__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of the current GPU's scratch array (NULL on failure).
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* z, const void* beta,
                                 float g_min, const float* s0, void* o, float* s_final, int B, int T, int H,
                                 int dk, int dv, int chunk, kda_dtype dt, void* stream) {
    const kda_status st = check_chunk_args(q, k, v, z, beta, g_min, s0, o, s_final, B, T, H, dk, dv, chunk, dt,
                                           nullptr);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    const size_t need = kda::chunk_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16);
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0 && !(ws = scratch_address())) return KDA_ERR_HIP;
    kda::ChunkArgs a{q, k, v, z, beta, g_min, s0, o, s_final, B, T, H, dk, dv, dt == KDA_BF16, ws, stream};
    return finish(kda::launch_chunk(a), stream);
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* z, const void* beta,
                              float g_min, float* state, void* o, int B, int H, int dk, int dv, kda_dtype dt,
                              void* stream) {
    const kda_status st = check_step_args(q, k, v, z, beta, g_min, state, B, H, dk, dv, dt);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (!o) return KDA_ERR_NULL;
    if (!aligned16(o)) return KDA_ERR_ALIGN;
    kda::DecodeArgs a{q, k, v, z, beta, g_min, state, o, B, H, dk, dv, dt == KDA_BF16, stream};
    return finish(kda::launch_decode(a), stream);
}

size_t kda_out_gate_workspace_bytes(int B, int T, int H, int dv, int d_model, kda_dtype dt,
                                    int with_projection) {
    if (B < 0 || T < 0 || H < 0 || !dim_ok(dv)) return 0;
    return kda::gate_workspace_bytes(B, T, H, dv, d_model, dt == KDA_BF16, with_projection != 0);
}

kda_status kda_out_gate(const void* o, const void* gate, float eps, const void* w, void* y, int B, int T,
                        int H, int dv, int d_model, kda_dtype dt, void* workspace, size_t workspace_bytes,
                        void* stream) {
    if (B < 0 || T < 0 || H < 0 || d_model < 0) return KDA_ERR_SHAPE;
    if (!dim_ok(dv) || (dt != KDA_F32 && dt != KDA_BF16)) return KDA_ERR_UNSUPPORTED;
    if (w && (dt != KDA_BF16 || d_model % 16 != 0 || d_model == 0)) return KDA_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || !isfinite(eps)) return KDA_ERR_ARG;
    const long long rows = (long long)B * T;
    if (rows * H > (1LL << 40)) return KDA_ERR_SHAPE;
    if (w && ((rows + 127) / 128 > 65535 || (long long)H * dv > (1 << 20))) return KDA_ERR_SHAPE;
    if (rows == 0 || H == 0) return KDA_OK;
    if (!o || !gate || !y) return KDA_ERR_NULL;
    if (!aligned16(o) || !aligned16(gate) || !aligned16(w) || !aligned16(y) || !aligned16(workspace))
        return KDA_ERR_ALIGN;
    const size_t need = kda::gate_workspace_bytes(B, T, H, dv, d_model, dt == KDA_BF16, w != nullptr);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    kda::GateArgs a{o, gate, eps, w, y, B, T, H, dv, d_model, dt == KDA_BF16, workspace, stream};
    return finish(kda::launch_out_gate(a), stream);
}

size_t kda_gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, kda_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || chunk != 64 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    if (dt != KDA_F32 && dt != KDA_BF16) return 0;
    // the channel-wise operator's workspace (256-byte aligned), then the
    // logits broadcast over the d_k channels
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const size_t base = (kda::chunk_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16) + 255) / 256 * 256;
    return base + (size_t)B * T * H * dk * esz;
}

kda_status kda_gdn_chunk_fwd(const void* q, const void* k, const void* v, const void* z, const void* beta,
                             float g_min, const float* s0, void* o, float* s_final, int B, int T, int H, int dk,
                             int dv, int chunk, kda_dtype dt, void* workspace, size_t workspace_bytes,
                             void* stream) {
    const kda_status st = check_chunk_args(q, k, v, z, beta, g_min, s0, o, s_final, B, T, H, dk, dv, chunk, dt,
                                           workspace);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    const size_t need = kda_gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dt);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const size_t zbytes = (size_t)B * T * H * dk * esz;
    const size_t base = need - zbytes;
    if (kda::chunk_scalar_gate_native(T, dk, dv, dt == KDA_BF16, g_min)) {
        // the pipelined kernels read the logit per (token, head) directly
        kda::ChunkArgs a{q, k, v, z, beta, g_min, s0, o, s_final, B, T, H, dk, dv, true,
                         base ? workspace : nullptr, stream};
        a.scalar_z = true;
        return finish(kda::launch_chunk(a), stream);
    }
    void* zfull = zbytes ? (unsigned char*)workspace + (need - zbytes) : nullptr;
    hipError_t err = kda::launch_broadcast_gate(z, zfull, (size_t)B * T * H, dk, dt == KDA_BF16, stream);
    if (err != hipSuccess) return finish(err, stream);
    kda::ChunkArgs a{q, k, v, zfull, beta, g_min, s0, o, s_final, B, T, H, dk, dv, dt == KDA_BF16,
                     base ? workspace : nullptr, stream};
    return finish(kda::launch_chunk(a), stream);
}

kda_status kda_gdn_recurrent_step(const void* q, const void* k, const void* v, const void* z, const void* beta,
                                  float g_min, float* state, void* o, int B, int H, int dk, int dv, kda_dtype dt,
                                  void* stream) {
    const kda_status st = check_step_args(q, k, v, z, beta, g_min, state, B, H, dk, dv, dt);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (!o) return KDA_ERR_NULL;
    if (!aligned16(o)) return KDA_ERR_ALIGN;
    kda::DecodeArgs a{q, k, v, z, beta, g_min, state, o, B, H, dk, dv, dt == KDA_BF16, stream};
    a.z_scalar = true;
    return finish(kda::launch_decode(a), stream);
}

size_t kda_recurrent_layer_step_workspace_bytes(int B, int H, int dv, int d_model, kda_dtype dt,
                                                int with_projection) {
    (void)dt;
    if (B < 0 || H < 0 || d_model < 0 || !dim_ok(dv) || !with_projection) return 0;
    // the gated row in bf16, 256-byte aligned, then the GEMM's scratch
    return ((size_t)B * H * dv * 2 + 255) / 256 * 256 + kda::projection_scratch_bytes(B, d_model, H * dv);
}

kda_status kda_recurrent_layer_step(const void* q, const void* k, const void* v, const void* z, const void* beta,
                                    float g_min, float* state, const void* gate, float eps, const void* w, void* o,
                                    void* y, int B, int H, int dk, int dv, int d_model, kda_dtype dt,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    // the projection's own checks first, in the order kda_out_gate makes them
    if (B < 0 || H < 0 || d_model < 0) return KDA_ERR_SHAPE;
    if (!dim_ok(dk) || !dim_ok(dv) || (dt != KDA_F32 && dt != KDA_BF16)) return KDA_ERR_UNSUPPORTED;
    if (w && (dt != KDA_BF16 || d_model % 16 != 0 || d_model == 0)) return KDA_ERR_UNSUPPORTED;
    if (w && ((B + 127) / 128 > 65535 || (long long)H * dv > (1 << 20))) return KDA_ERR_SHAPE;
    if (!(eps >= 0.f) || !isfinite(eps)) return KDA_ERR_ARG;
    const kda_status st = check_step_args(q, k, v, z, beta, g_min, state, B, H, dk, dv, dt);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (!gate || !y) return KDA_ERR_NULL;
    if (!aligned16(gate) || !aligned16(w) || !aligned16(o) || !aligned16(y) || !aligned16(workspace))
        return KDA_ERR_ALIGN;
    const size_t need = kda_recurrent_layer_step_workspace_bytes(B, H, dv, d_model, dt, w != nullptr);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    kda::DecodeArgs a{q, k, v, z, beta, g_min, state, o, B, H, dk, dv, dt == KDA_BF16, stream};
    a.gate = gate;
    a.eps = eps;
    a.y = w ? workspace : y;
    a.y_bf16 = w != nullptr;
    hipError_t err = kda::launch_decode(a);
    if (err == hipSuccess && w) {
        void* lws = (unsigned char*)workspace + ((size_t)B * H * dv * 2 + 255) / 256 * 256;
        err = kda::launch_projection(workspace, w, y, B, d_model, H * dv, lws, stream);
    }
    return finish(err, stream);
}

}  // extern "C"

namespace {

// Workspace of kda_chunk_layer_fwd: the prefill's (256-byte aligned); then,
// when the epilogue is not fused into the prefill kernels, room for o; then
// the epilogue's (the gated rows in bf16 and the GEMM scratch, with a
// projection only).
struct LayerWs {
    size_t chunk, obuf, gate, total;
};
LayerWs layer_ws(int B, int T, int H, int dk, int dv, int d_model, kda_dtype dt, bool proj) {
    const bool bf = dt == KDA_BF16;
    LayerWs r;
    r.chunk = (kda::chunk_workspace_bytes(B, T, H, dk, dv, bf) + 255) / 256 * 256;
    r.obuf = kda::chunk_gate_fused(B, T, H, dk, dv, bf) ? 0 : ((size_t)B * T * H * dv * (bf ? 2 : 4) + 255) / 256 * 256;
    r.gate = kda::gate_workspace_bytes(B, T, H, dv, d_model, bf, proj);
    r.total = r.chunk + r.obuf + r.gate;
    return r;
}

}  // namespace

extern "C" {

size_t kda_chunk_layer_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int d_model,
                                           kda_dtype dt, int with_projection) {
    if (B < 0 || T < 0 || H < 0 || d_model < 0 || chunk != 64 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    if (dt != KDA_F32 && dt != KDA_BF16) return 0;
    return layer_ws(B, T, H, dk, dv, d_model, dt, with_projection != 0).total;
}

kda_status kda_chunk_layer_fwd(const void* q, const void* k, const void* v, const void* z, const void* beta,
                               float g_min, const float* s0, const void* gate, float eps, const void* w, void* o,
                               void* y, float* s_final, int B, int T, int H, int dk, int dv, int chunk,
                               int d_model, kda_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
    // the epilogue's own checks first, in the order kda_out_gate makes them
    if (B < 0 || T < 0 || H < 0 || d_model < 0) return KDA_ERR_SHAPE;
    if (!dim_ok(dv) || (dt != KDA_F32 && dt != KDA_BF16)) return KDA_ERR_UNSUPPORTED;
    if (w && (dt != KDA_BF16 || d_model % 16 != 0 || d_model == 0)) return KDA_ERR_UNSUPPORTED;
    if (w && (((long long)B * T + 127) / 128 > 65535 || (long long)H * dv > (1 << 20))) return KDA_ERR_SHAPE;
    if (!(eps >= 0.f) || !isfinite(eps)) return KDA_ERR_ARG;
    // then the prefill's, with y in the place of the required output
    const kda_status st = check_chunk_args(q, k, v, z, beta, g_min, s0, y, s_final, B, T, H, dk, dv, chunk, dt,
                                           workspace);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (T > 0 && !gate) return KDA_ERR_NULL;
    if (!aligned16(gate) || !aligned16(w) || !aligned16(o)) return KDA_ERR_ALIGN;
    const LayerWs ws = layer_ws(B, T, H, dk, dv, d_model, dt, w != nullptr);
    if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return KDA_ERR_WORKSPACE;
    unsigned char* wsb = (unsigned char*)workspace;
    void* chunk_ws = ws.chunk ? wsb : nullptr;
    void* gate_ws = ws.gate ? wsb + ws.chunk + ws.obuf : nullptr;
    const bool bf = dt == KDA_BF16;
    kda::ChunkArgs a{q, k, v, z, beta, g_min, s0, o, s_final, B, T, H, dk, dv, bf, chunk_ws, stream};
    hipError_t err;
    if (T > 0 && (g_min < kda::CHUNK_G_MIN_LIMIT || kda::chunk_gate_fused(B, T, H, dk, dv, bf))) {
        // y, or with a projection its bf16 input rows, from the prefill kernels
        // (the token-sequential kernel for g_min below the chunkwise limit)
        a.gate = gate;
        a.eps = eps;
        a.y = w ? gate_ws : y;
        err = kda::launch_chunk(a);
        if (err == hipSuccess && w) {
            const size_t ybytes = ws.gate - kda::projection_scratch_bytes(B * T, d_model, H * dv);
            err = kda::launch_projection(gate_ws, w, y, B * T, d_model, H * dv, (unsigned char*)gate_ws + ybytes,
                                         stream);
        }
        return finish(err, stream);
    }
    // other sizes: the prefill into o (or the workspace), then the epilogue
    if (!a.o) a.o = wsb + ws.chunk;
    err = kda::launch_chunk(a);
    if (err == hipSuccess && T > 0) {
        kda::GateArgs g{a.o, gate, eps, w, y, B, T, H, dv, d_model, bf, gate_ws, stream};
        err = kda::launch_out_gate(g);
    }
    return finish(err, stream);
}

}  // extern "C"

extern "C" {

size_t kda_recurrent_bwd_workspace_bytes(int B, int T, int H, int dk, int dv) {
    if (B < 0 || T < 0 || H < 0 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    return kda::bwd_workspace_bytes(B, T, H, dk, dv);
}

kda_status kda_recurrent_bwd(const void* q, const void* k, const void* v, const void* z, const void* beta,
                             float g_min, const float* s0, const void* grad_o, const float* grad_s_final,
                             float* grad_q, float* grad_k, float* grad_v, float* grad_z, float* grad_beta,
                             float* grad_s0, int B, int T, int H, int dk, int dv, kda_dtype dt, void* workspace,
                             size_t workspace_bytes, void* stream) {
    // the prefill's checks on the forward inputs (grad_o in the output's place)
    const kda_status st = check_chunk_args(q, k, v, z, beta, g_min, s0, grad_o, grad_s_final, B, T, H, dk, dv, 64,
                                           dt, workspace);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (T > 0 && (!grad_q || !grad_k || !grad_v || !grad_z || !grad_beta)) return KDA_ERR_NULL;
    if (!aligned16(grad_q) || !aligned16(grad_k) || !aligned16(grad_v) || !aligned16(grad_z) ||
        !aligned16(grad_beta) || !aligned16(grad_s0))
        return KDA_ERR_ALIGN;
    const size_t need = kda::bwd_workspace_bytes(B, T, H, dk, dv);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    kda::BwdArgs a{q, k, v, z, beta, g_min, s0, grad_o, grad_s_final, grad_q, grad_k, grad_v, grad_z, grad_beta,
                   grad_s0, B, T, H, dk, dv, dt == KDA_BF16, workspace, stream};
    if (T == 0 && !grad_s0) return KDA_OK;
    return finish(kda::launch_bwd(a), stream);
}

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, kda_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || chunk != 64 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    if (dt != KDA_F32 && dt != KDA_BF16) return 0;
    return kda::chunk_bwd_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16);
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* z, const void* beta, float g_min,
                         const float* s0, const void* grad_o, const float* grad_s_final, float* grad_q,
                         float* grad_k, float* grad_v, float* grad_z, float* grad_beta, float* grad_s0, int B, int T,
                         int H, int dk, int dv, int chunk, kda_dtype dt, void* workspace, size_t workspace_bytes,
                         void* stream) {
    const kda_status st = check_chunk_args(q, k, v, z, beta, g_min, s0, grad_o, grad_s_final, B, T, H, dk, dv, chunk,
                                           dt, workspace);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (T > 0 && (!grad_q || !grad_k || !grad_v || !grad_z || !grad_beta)) return KDA_ERR_NULL;
    if (!aligned16(grad_q) || !aligned16(grad_k) || !aligned16(grad_v) || !aligned16(grad_z) ||
        !aligned16(grad_beta) || !aligned16(grad_s0))
        return KDA_ERR_ALIGN;
    const size_t need = kda::chunk_bwd_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    kda::BwdArgs a{q, k, v, z, beta, g_min, s0, grad_o, grad_s_final, grad_q, grad_k, grad_v, grad_z, grad_beta,
                   grad_s0, B, T, H, dk, dv, dt == KDA_BF16, workspace, stream};
    if (T == 0 && !grad_s0) return KDA_OK;
    return finish(kda::launch_chunk_bwd(a), stream);
}

kda_status kda_dplr_fwd(const void* q, const void* k, const void* v, const void* z, const void* a, const void* b,
                        float g_min, const float* s0, void* o, float* s_final, int B, int T, int H, int dk, int dv,
                        kda_dtype dt, void* stream) {
    // the prefill's checks, with a in beta's place, then those of b
    const kda_status st = check_chunk_args(q, k, v, z, a, g_min, s0, o, s_final, B, T, H, dk, dv, 64, dt, nullptr);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (T > 0 && !b) return KDA_ERR_NULL;
    if (!aligned16(b)) return KDA_ERR_ALIGN;
    if (T == 0 && !s_final) return KDA_OK;
    kda::DplrArgs x{q, k, v, z, a, b, g_min, s0, o, s_final, B, T, H, dk, dv, dt == KDA_BF16, false, stream};
    return finish(kda::launch_dplr(x), stream);
}

size_t kda_dplr_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, kda_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || chunk != 64 || !dim_ok(dk) || !dim_ok(dv)) return 0;
    if (dt != KDA_F32 && dt != KDA_BF16) return 0;
    return kda::dplr_chunk_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16);
}

kda_status kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* z, const void* a,
                              const void* b, float g_min, const float* s0, void* o, float* s_final, int B, int T,
                              int H, int dk, int dv, int chunk, kda_dtype dt, void* workspace,
                              size_t workspace_bytes, void* stream) {
    const kda_status st = check_chunk_args(q, k, v, z, a, g_min, s0, o, s_final, B, T, H, dk, dv, chunk, dt,
                                           workspace);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (T > 0 && !b) return KDA_ERR_NULL;
    if (!aligned16(b)) return KDA_ERR_ALIGN;
    if (T == 0 && !s_final) return KDA_OK;
    const bool chunked = T > 0 && g_min >= KDA_CHUNK_G_MIN_LIMIT;
    const size_t need = chunked ? kda::dplr_chunk_workspace_bytes(B, T, H, dk, dv, dt == KDA_BF16) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    kda::DplrArgs x{q, k, v, z, a, b, g_min, s0, o, s_final, B, T, H, dk, dv, dt == KDA_BF16, false, stream};
    return finish(kda::launch_dplr_chunk(x, workspace), stream);
}

kda_status kda_dplr_recurrent_step(const void* q, const void* k, const void* v, const void* z, const void* a,
                                   const void* b, float g_min, float* state, void* o, int B, int H, int dk, int dv,
                                   kda_dtype dt, void* stream) {
    const kda_status st = check_step_args(q, k, v, z, a, g_min, state, B, H, dk, dv, dt);
    if (st != KDA_OK || B == 0 || H == 0) return st;
    if (!b || !o) return KDA_ERR_NULL;
    if (!aligned16(b) || !aligned16(o)) return KDA_ERR_ALIGN;
    kda::DplrArgs x{q, k, v, z, a, b, g_min, nullptr, o, state, B, 1, H, dk, dv, dt == KDA_BF16, true, stream};
    return finish(kda::launch_dplr(x), stream);
}

}  // extern "C"
