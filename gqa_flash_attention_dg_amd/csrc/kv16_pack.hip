// kv16_pack.hip -- dg_pack_kv16: f32 -> 16-bit storage for K and V on gfx950.
//
// inferencelayer 0.2.8, src/deepencoder_gpu.rs, `flash_reg_kv16_src`: the flash reads its keys
// and values from an f16 copy of its inputs made by a separate packing pass, widening each to f32
// before the unchanged f32 math.  This is that pack pass, for IEEE binary16 or bfloat16, both
// rounded to nearest with ties to even.  HBM-bound: each thread turns 8 floats (two 16-byte
// loads) into one 16-byte store.
#include "kv16.hpp"

namespace {

using dg::to_bf16;
using dg::to_f16;

template <int kFmt>
__device__ inline uint32_t pack2(float a, float b) {
    return kFmt == DG_KV_F16 ? (to_f16(a) | (to_f16(b) << 16)) : (to_bf16(a) | (to_bf16(b) << 16));
}

template <int kFmt>
__global__ void __launch_bounds__(256) pack_kv16_kernel(const float* __restrict__ src,
                                                        uint16_t* __restrict__ dst, size_t n) {
    const size_t i0 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= n) return;
    if (i0 + 8 <= n) {
        const float4 a = *reinterpret_cast<const float4*>(src + i0);
        const float4 b = *reinterpret_cast<const float4*>(src + i0 + 4);
        *reinterpret_cast<uint4*>(dst + i0) =
            make_uint4(pack2<kFmt>(a.x, a.y), pack2<kFmt>(a.z, a.w), pack2<kFmt>(b.x, b.y),
                       pack2<kFmt>(b.z, b.w));
    } else {
        for (size_t i = i0; i < n; ++i)
            dst[i] = (uint16_t)(kFmt == DG_KV_F16 ? to_f16(src[i]) : to_bf16(src[i]));
    }
}

}  // namespace

extern "C" int dg_pack_kv16(const float* src, void* dst, size_t n, int format, void* stream) {
    const char* fn = "dg_pack_kv16";
    if (format != DG_KV_F16 && format != DG_KV_BF16)
        return dg::fail(DG_EINVAL, "%s: format must be DG_KV_F16 or DG_KV_BF16, got %d", fn, format);
    if (n == 0) return dg::ok();
    if (!src || !dst) return dg::fail(DG_EINVAL, "%s: src and dst must be non-NULL", fn);
    if (n > (SIZE_MAX / 8)) return dg::fail(DG_EINVAL, "%s: size overflow", fn);
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
        return dg::fail(DG_EINVAL, "%s: src and dst must be 16-byte aligned", fn);
    if (dg::Span(src, n * 4).overlaps(dg::Span(dst, n * 2)))
        return dg::fail(DG_EINVAL, "%s: dst overlaps src", fn);
    const size_t threads = (n + 7) / 8;
    const size_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffULL) return dg::fail(DG_EUNSUPPORTED, "%s: too many elements", fn);
    hipStream_t s = (hipStream_t)stream;
    uint16_t* d = static_cast<uint16_t*>(dst);
    if (format == DG_KV_F16)
        hipLaunchKernelGGL(pack_kv16_kernel<DG_KV_F16>, dim3((unsigned)blocks), dim3(256), 0, s, src, d, n);
    else
        hipLaunchKernelGGL(pack_kv16_kernel<DG_KV_BF16>, dim3((unsigned)blocks), dim3(256), 0, s, src, d, n);
    return dg::launch_status(fn);
}
