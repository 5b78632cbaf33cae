// conversions.hip -- test-only kernels that apply the epilogue library's own
// conversion helpers (quant_epilogues_amd/csrc/dit_device.h) to sweeps of
// inputs, so that the tests can compare them with the CPU oracle's encoders.
// Not part of the product library; built next to this file by the build step.
//
// dit_cvt_sweep(kind, in, out, n, stream), on device buffers:
//   kind 0: out[i] (u32)  = 4 E4M3 bytes of clamp_e4m3(in[4i..4i+3])  (n % 4 == 0)
//   kind 1: out[i] (u32)  = 8 E2M1 nibbles of in[8i..8i+7]             (n % 8 == 0)
//   kind 2: out[i] (u32)  = 2 bf16 of in[2i], in[2i+1] (pack_bf16)     (n % 2 == 0)
//   kind 3: out[i] (f32)  = round_bf16(in[i])
//   kind 4: out[i] (f32)  = div6_bf16(in[i])
// Returns 0, or -1 for an unknown kind or a size it does not take, or the HIP
// error of the launch.
// dit_div6_host(in, out, n): div6_bf16 compiled for the host, on host buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dit_device.h"

namespace {

__global__ void cvt_kernel(int kind, const float* __restrict__ in, void* __restrict__ out,
                           int64_t units) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= units) return;
    uint32_t* o32 = static_cast<uint32_t*>(out);
    float* of = static_cast<float*>(out);
    if (kind == 0) {
        const float* p = in + 4 * i;
        o32[i] = dit::pack_e4m3x4(dit::clamp_e4m3(p[0]), dit::clamp_e4m3(p[1]),
                                  dit::clamp_e4m3(p[2]), dit::clamp_e4m3(p[3]));
    } else if (kind == 1) {
        const float* p = in + 8 * i;
        const float t[8] = {p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
        o32[i] = dit::pack_e2m1x8(t);
    } else if (kind == 2) {
        o32[i] = dit::pack_bf16(in[2 * i], in[2 * i + 1]);
    } else if (kind == 3) {
        of[i] = dit::round_bf16(in[i]);
    } else {
        of[i] = dit::div6_bf16(in[i]);
    }
}

}  // namespace

extern "C" int dit_cvt_sweep(int kind, const float* in, void* out, int64_t n, void* stream) {
    static const int per_unit[5] = {4, 8, 2, 1, 1};
    if (kind < 0 || kind > 4 || n < 0 || n % per_unit[kind] != 0 || n > (int64_t(1) << 31))
        return -1;
    const int64_t units = n / per_unit[kind];
    if (units == 0) return 0;
    hipLaunchKernelGGL(cvt_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), kind, in, out, units);
    return (int)hipGetLastError();
}

extern "C" void dit_div6_host(const float* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = dit::div6_bf16(in[i]);
}
