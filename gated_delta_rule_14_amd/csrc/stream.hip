// stream.hip -- kda_stream_scale: x <- s * x in place over a device buffer of
// fp32, the memory access pattern of the decode step's state (every byte read
// once and written once, 16-byte accesses).  It measures the read-modify-write
// rate this GPU's HBM sustains, the practical ceiling of kda_recurrent_step.
//
// Each thread moves U float4 per pass: all U loads are issued before the
// first store, so U * 16 bytes per thread are in flight.  NT selects
// non-temporal loads and stores (the decode step uses them: the state does not
// fit the caches and is not reused within a step).
#include "../../include/kda.h"
#include "kda_device.hpp"

namespace kda {
namespace {

template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_scale_kernel(f32x4* __restrict__ x, size_t n4, float s) {
    const size_t stride = (size_t)gridDim.x * 256 * U;
    for (size_t base = (size_t)blockIdx.x * 256 * U + threadIdx.x; base < n4; base += stride) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = base + (size_t)u * 256;
            if (i < n4) v[u] = NT ? __builtin_nontemporal_load(x + i) : x[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = base + (size_t)u * 256;
            if (i < n4) {
                if (NT)
                    __builtin_nontemporal_store(v[u] * s, x + i);
                else
                    x[i] = v[u] * s;
            }
        }
    }
}

template <int U, bool NT>
hipError_t launch(float* x, size_t n4, float s, int waves_per_cu, hipStream_t st) {
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    // workgroups of 4 waves: waves_per_cu / 4 per compute unit, or one pass
    size_t wg = (size_t)cus * (waves_per_cu > 0 ? (waves_per_cu + 3) / 4 : 1);
    const size_t need = (n4 + 256 * U - 1) / (256 * U);
    if (waves_per_cu <= 0 || wg > need) wg = need;
    if (wg == 0) return hipSuccess;
    hipLaunchKernelGGL((stream_scale_kernel<U, NT>), dim3((unsigned)wg), dim3(256), 0, st, (f32x4*)x, n4, s);
    return hipGetLastError();
}

}  // namespace
}  // namespace kda

extern "C" kda_status kda_stream_scale(float* x, size_t n, float s, int variant, void* stream) {
    if (n == 0) return KDA_OK;
    if (!x) return KDA_ERR_NULL;
    if (((uintptr_t)x & 15u) != 0 || n % 4 != 0) return KDA_ERR_ALIGN;
    const size_t n4 = n / 4;
    hipStream_t st = (hipStream_t)stream;
    hipError_t err;
    // variant: bits 0-1 select U in {1, 2, 4, 8}; bit 2 non-temporal;
    // bits 3.. the waves per compute unit of a grid-stride launch (0: one pass)
    const int u = variant & 3, wpc = variant >> 3;
    const bool nt = (variant & 4) != 0;
    switch (u) {
        case 0: err = nt ? kda::launch<1, true>(x, n4, s, wpc, st) : kda::launch<1, false>(x, n4, s, wpc, st); break;
        case 1: err = nt ? kda::launch<2, true>(x, n4, s, wpc, st) : kda::launch<2, false>(x, n4, s, wpc, st); break;
        case 2: err = nt ? kda::launch<4, true>(x, n4, s, wpc, st) : kda::launch<4, false>(x, n4, s, wpc, st); break;
        default: err = nt ? kda::launch<8, true>(x, n4, s, wpc, st) : kda::launch<8, false>(x, n4, s, wpc, st); break;
    }
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
