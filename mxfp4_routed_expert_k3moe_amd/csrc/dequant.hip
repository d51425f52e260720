// dequant.hip -- decode an MXFP4 matrix to fp32 or bf16 with the device helpers the
// matrix kernels use (colibri PR #684, MXFP4-kernel commit: packed [O, I/2] bytes,
// low nibble = even column, bit3 = sign; scales [O, I/32]; w = v * 2^(s-127)).
// One thread per 16-byte chunk (32 codes, one scale byte).
#include "device.hpp"
#include "launch.hpp"

namespace k3moe {

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q,
                                                      const uint8_t* __restrict__ s, int O, int I,
                                                      void* __restrict__ out) {
    const int nch = I >> 5;
    const size_t total = (size_t)O * nch;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
        const size_t o = c / nch, ch = c % nch;
        const uint4 qv = *reinterpret_cast<const uint4*>(q + o * (size_t)(I >> 1) + ch * 16);
        const uint32_t sc = s[o * (size_t)nch + ch];
        const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
        if (BF16) {
            uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o * (size_t)I + ch * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 v = fp4x8_to_bf16(words[j], sc);
                dst[j] = make_uint4(v.x, v.y, v.z, v.w);
            }
        } else {
            float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + o * (size_t)I + ch * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v[8];
                fp4x8_to_f32(words[j], sc, v);
                dst[2 * j] = make_float4(v[0], v[1], v[2], v[3]);
                dst[2 * j + 1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
    }
}

}  // namespace

hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int O, int I, void* out, int out_bf16,
                          hipStream_t stream) {
    const size_t total = (size_t)O * (I >> 5);
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (out_bf16)
        hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, q, s, O, I, out);
    else
        hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, q, s, O, I, out);
    return hipGetLastError();
}

}  // namespace k3moe
