// Measurement probes (include/fa_probe.h): register-only loops that keep one
// execution unit busy, to measure on the device the rates the attention
// kernels are held against -- the MFMA rate per input type, v_exp_f32 and
// fp32 FMA throughput -- and the shader clock while they run.
//
// Every wave runs NCH independent dependency chains, so that consecutive
// instructions never wait for each other; the chains' values are summed and
// stored at the end so that the loop cannot be removed.
#include <hip/hip_runtime.h>
#include <string.h>

#include "fa_device.h"
#include "../../include/fa.h"
#include "../../include/fa_probe.h"

namespace fa {
namespace {

constexpr int kThreads = 256;  // 4 waves

template <int KIND> struct MfmaOp;
template <> struct MfmaOp<FA_PROBE_MFMA_BF16> {
    typedef bf16x8 V;
    typedef f32x16 A;
    static constexpr int NCH = 8;
    static constexpr double FLOP = 2.0 * 32 * 32 * 16;
    static __device__ V operand(int lane) {
        V v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)(1e-3f * (float)((lane + e) & 7));
        return v;
    }
    static __device__ A mma(V a, V b, A c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};
template <> struct MfmaOp<FA_PROBE_MFMA_F16> {
    typedef f16x8 V;
    typedef f32x16 A;
    static constexpr int NCH = 8;
    static constexpr double FLOP = 2.0 * 32 * 32 * 16;
    static __device__ V operand(int lane) {
        V v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (_Float16)(1e-3f * (float)((lane + e) & 7));
        return v;
    }
    static __device__ A mma(V a, V b, A c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};
template <> struct MfmaOp<FA_PROBE_MFMA_FP8> {
    typedef i32x8 V;
    typedef f32x16 A;
    static constexpr int NCH = 8;
    static constexpr double FLOP = 2.0 * 32 * 32 * 64;
    static __device__ V operand(int lane) {
        V v;
        // E4M3 codes 0x18..0x1f (small normal numbers), four per register
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (int)(0x18181818u + 0x01010101u * (unsigned)((lane + e) & 7));
        return v;
    }
    static __device__ A mma(V a, V b, A c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};
template <> struct MfmaOp<FA_PROBE_MFMA_F32> {
    typedef float V;
    typedef f32x16 A;
    static constexpr int NCH = 8;
    static constexpr double FLOP = 2.0 * 32 * 32 * 2;
    static __device__ V operand(int lane) { return 1e-3f * (float)(lane & 7); }
    static __device__ A mma(V a, V b, A c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }
};

__device__ __forceinline__ void record_clocks(uint64_t *clocks, uint64_t c0, uint64_t w0) {
    const uint64_t c1 = clock64(), w1 = wall_clock64();
    if (clocks && lane_id() == 0) {
        const int64_t slot = 2 * ((int64_t)blockIdx.x * (kThreads / 64) + wave_id());
        clocks[slot] = c1 - c0;
        clocks[slot + 1] = w1 - w0;
    }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int64_t iters, float *sink, uint64_t *clocks) {
    typedef MfmaOp<KIND> Op;
    const int lane = lane_id();
    const typename Op::V a = Op::operand(lane), b = Op::operand(lane + 3);
    typename Op::A acc[Op::NCH];
#pragma unroll
    for (int i = 0; i < Op::NCH; ++i) acc[i] = (typename Op::A){};
    const uint64_t c0 = clock64(), w0 = wall_clock64();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < Op::NCH; ++i) acc[i] = Op::mma(a, b, acc[i]);
    }
    record_clocks(clocks, c0, w0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < Op::NCH; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

constexpr int kValuChains = 16;

// KIND == FA_PROBE_EXP: x <- 2^-x per chain (stays in (0, 1]); FA_PROBE_FMA:
// x <- x * a + b.
template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_probe_kernel(int64_t iters, float *sink, uint64_t *clocks) {
    const int lane = lane_id();
    float x[kValuChains];
#pragma unroll
    for (int i = 0; i < kValuChains; ++i) x[i] = 1e-3f * (float)(lane + i);
    const float fa_ = 0.999f + 1e-6f * (float)(lane & 3), fb = 1e-3f * (float)(1 + (lane & 1));
    const uint64_t c0 = clock64(), w0 = wall_clock64();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kValuChains; ++i) {
            if constexpr (KIND == FA_PROBE_EXP)
                x[i] = __builtin_amdgcn_exp2f(-x[i]);
            else
                x[i] = __builtin_fmaf(x[i], fa_, fb);
        }
    }
    record_clocks(clocks, c0, w0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kValuChains; ++i) s += x[i];
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Streaming read of n16 16-byte chunks at a: thread t of the T threads of
// the grid reads chunks t, t + T, t + 2T, ..., eight at a time in flight
// (non-temporal: the data is read once), and stores the low 16 bits of the
// xor of the words it read, as an exact float.
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4 *__restrict__ a, int64_t n16, float *sink) {
    constexpr int U = 8;
    const int64_t T = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * T < n16; i += U * T) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(a + i + u * T);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += T) acc ^= __builtin_nontemporal_load(a + i);
    const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = (float)(x & 0xFFFFu);
}

bool on_gfx950() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
    return strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

}  // namespace
}  // namespace fa

extern "C" double fa_probe_work_per_iter(int kind) {
    using namespace fa;
    switch (kind) {
        case FA_PROBE_MFMA_BF16: return MfmaOp<FA_PROBE_MFMA_BF16>::FLOP * MfmaOp<FA_PROBE_MFMA_BF16>::NCH;
        case FA_PROBE_MFMA_F16: return MfmaOp<FA_PROBE_MFMA_F16>::FLOP * MfmaOp<FA_PROBE_MFMA_F16>::NCH;
        case FA_PROBE_MFMA_FP8: return MfmaOp<FA_PROBE_MFMA_FP8>::FLOP * MfmaOp<FA_PROBE_MFMA_FP8>::NCH;
        case FA_PROBE_MFMA_F32: return MfmaOp<FA_PROBE_MFMA_F32>::FLOP * MfmaOp<FA_PROBE_MFMA_F32>::NCH;
        case FA_PROBE_EXP:
        case FA_PROBE_FMA: return 64.0 * kValuChains;
        default: return 0.0;
    }
}

extern "C" int64_t fa_probe_wall_clock_khz(void) {
    int dev = -1, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz > 0 ? khz : 0;
}

extern "C" int fa_probe_hbm_read(const void *buf, int64_t bytes, int64_t n_wg, float *sink, void *stream) {
    using namespace fa;
    if (n_wg < 1 || n_wg > (1 << 20) || bytes < 16 || bytes % 16) return FA_ERR_SHAPE;
    if (!buf || !sink) return FA_ERR_NULL;
    if ((uintptr_t)buf % 16 || (uintptr_t)sink % alignof(float)) return FA_ERR_ALIGN;
    if (!on_gfx950()) return FA_ERR_DEVICE;
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)n_wg), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_probe(int kind, int64_t n_wg, int64_t iters, float *sink, uint64_t *clocks, void *stream) {
    using namespace fa;
    if (kind < FA_PROBE_MFMA_BF16 || kind > FA_PROBE_FMA) return FA_ERR_DTYPE;
    if (n_wg < 1 || n_wg > (1 << 20) || iters < 1 || iters > (1 << 30)) return FA_ERR_SHAPE;
    if (!sink) return FA_ERR_NULL;
    if ((uintptr_t)sink % alignof(float) || (uintptr_t)clocks % alignof(uint64_t)) return FA_ERR_ALIGN;
    if (!on_gfx950()) return FA_ERR_DEVICE;
    const dim3 grid((unsigned)n_wg), block(kThreads);
    hipStream_t s = (hipStream_t)stream;
    switch (kind) {
        case FA_PROBE_MFMA_BF16: hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_BF16>, grid, block, 0, s, iters, sink, clocks); break;
        case FA_PROBE_MFMA_F16: hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_F16>, grid, block, 0, s, iters, sink, clocks); break;
        case FA_PROBE_MFMA_FP8: hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_FP8>, grid, block, 0, s, iters, sink, clocks); break;
        case FA_PROBE_MFMA_F32: hipLaunchKernelGGL(mfma_probe_kernel<FA_PROBE_MFMA_F32>, grid, block, 0, s, iters, sink, clocks); break;
        case FA_PROBE_EXP: hipLaunchKernelGGL(valu_probe_kernel<FA_PROBE_EXP>, grid, block, 0, s, iters, sink, clocks); break;
        default: hipLaunchKernelGGL(valu_probe_kernel<FA_PROBE_FMA>, grid, block, 0, s, iters, sink, clocks); break;
    }
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
