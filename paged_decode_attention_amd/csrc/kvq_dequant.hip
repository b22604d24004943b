// Dequantize one page of the K or V half of the cache to float32, optionally mapping it back
// to the original basis with R^T (= R). Inspection path; the attention kernel never
// materialises these values.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

template <int BITS>
__global__ __launch_bounds__(64) void dequant_page_kernel(const DequantArgs a) {
  constexpr int kRow = kHeadDim * BITS / 8;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const int lane = threadIdx.x;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int h = blockIdx.x;
  const int ps = a.page_size;
  const int64_t tile = static_cast<int64_t>(a.page) * a.num_kv_heads + h;
  const uint8_t* base = a.codes + tile * ps * kRow;
  const float2* sz = reinterpret_cast<const float2*>(a.sz) + tile * ps;
  for (int it = 0; it < ps / 4; ++it) {
    const int off = it * 4 + grp;
    uint32_t codes = 0;
    if (a.tensor == 0) {
      codes = (BITS == 4) ? *reinterpret_cast<const uint32_t*>(base + off * kRow + li * 4)
                          : *reinterpret_cast<const uint16_t*>(base + off * kRow + li * 2);
    } else {
      // V tile: byte j of token t at ((t / 4) * row + j) * 4 + t % 4
      const uint8_t* p = base + ((off >> 2) * kRow) * 4 + (off & 3);
      constexpr int kBytes = BITS;  // bytes per lane: 8 codes * BITS / 8
#pragma unroll
      for (int m = 0; m < kBytes; ++m) codes |= static_cast<uint32_t>(p[(li * kBytes + m) * 4]) << (8 * m);
    }
    const float2 s = sz[off];
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(static_cast<float>((codes >> (BITS * k)) & kMask), s.x, s.y);
    if (a.unrotate) {
      fwht_row16(x, a.hb, li);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] *= a.inv_sqrt_hb;
    }
    float4* dst = reinterpret_cast<float4*>(a.out + (static_cast<int64_t>(h) * ps + off) * kHeadDim + li * 8);
    dst[0] = make_float4(x[0], x[1], x[2], x[3]);
    dst[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.num_kv_heads)), block(64);
  if (a.bits == 4) {
    hipLaunchKernelGGL(dequant_page_kernel<4>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(dequant_page_kernel<2>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvq
