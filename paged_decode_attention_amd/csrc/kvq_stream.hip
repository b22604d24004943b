// Streaming probes: how fast HBM serves a launch of a given shape that only moves bytes. A grid-
// stride loop over 16-byte units arranged in rows of read_units loads then write_units stores
// (the interface is described in kvq_stream.h).
#include "kvq_stream.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Unit u of the launch belongs to row u / per and is unit u mod per of that row. The division is a
// multiply by m = ceil(2^32 / per) (at most 2^32) and a shift: with e = m per - 2^32 in [0, per),
// u m / 2^32 = u / per + u e / (per 2^32), and the second term is below 1 for u < 2^32, so the
// quotient is exact or one too large; the remainder's sign shows which.
// Each thread takes kUnroll units a grid stride apart per iteration and issues all their loads
// before it uses any, so that every wave keeps several loads in flight.
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(1024) stream_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            uint32_t n_units, uint32_t per, uint64_t m,
                                                            uint32_t read_units, uint32_t write_units, uint32_t key,
                                                            uint32_t* sink) {
  const uint32_t stride = gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < n_units; base += kUnroll * stride) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t u = base + j * stride;
      uint32_t row = static_cast<uint32_t>((static_cast<uint64_t>(u) * m) >> 32);
      uint32_t k = u - row * per;
      if (static_cast<int32_t>(k) < 0) {  // quotient one too large
        --row;
        k += per;
      }
      x[j] = u32x4{0, 0, 0, 0};
      if (u < n_units) {
        if (k < read_units)
          x[j] = __builtin_nontemporal_load(src + static_cast<uint64_t>(row) * read_units + k);
        else
          dst[static_cast<uint64_t>(row) * write_units + (k - read_units)] = u32x4{u, row, k, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= x[j].x ^ x[j].y ^ x[j].z ^ x[j].w;
  }
  if (acc == key) *sink = acc;
}

// The split layout: of every read_units + write_units consecutive workgroups, the first read_units
// only read and the others only write, each kind walking its own linear stream (reads over
// rows * read_units units, writes over rows * write_units) with a grid stride over the workgroups
// of its kind. Each kind has the same share of the workgroups as of the bytes, so both streams end
// together and the chip sees the mix throughout.
__global__ void __launch_bounds__(1024) stream_probe_split_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst, uint32_t n_read,
                                                                  uint32_t n_write, uint32_t read_units,
                                                                  uint32_t write_units, uint32_t key, uint32_t* sink) {
  const uint32_t per = read_units + write_units;
  const uint32_t b = blockIdx.x;
  const uint32_t slot = b % per, group = b / per;
  const uint32_t groups_full = gridDim.x / per, tail = gridDim.x % per;
  // workgroups of this kind: read_units (write_units) per full group, and those of the last,
  // partial group that fall on this kind's slots
  const bool reader = slot < read_units;
  const uint32_t kind_blocks = reader ? groups_full * read_units + min(tail, read_units)
                                      : groups_full * write_units + (tail > read_units ? tail - read_units : 0);
  const uint32_t rank = reader ? group * read_units + slot : group * write_units + (slot - read_units);
  const uint32_t stride = kind_blocks * blockDim.x;
  const uint32_t n = reader ? n_read : n_write;
  uint32_t acc = 0;
  for (uint32_t base = rank * blockDim.x + threadIdx.x; base < n; base += kUnroll * stride) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t u = base + j * stride;
      x[j] = u32x4{0, 0, 0, 0};
      if (u < n) {
        if (reader)
          x[j] = __builtin_nontemporal_load(src + u);
        else
          dst[u] = u32x4{u / write_units, read_units + u % write_units, u, 1};
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= x[j].x ^ x[j].y ^ x[j].z ^ x[j].w;
  }
  if (acc == key) *sink = acc;
}

}  // namespace

extern "C" int32_t kvq_stream_probe(const void* src, void* dst, uint64_t rows, uint32_t read_units,
                                    uint32_t write_units, int32_t layout, uint32_t grid_blocks, uint32_t block_threads,
                                    uint32_t key, uint32_t* sink, hipStream_t stream) {
  const uint64_t per = static_cast<uint64_t>(read_units) + write_units;
  if (per == 0 || rows == 0 || grid_blocks == 0 || block_threads == 0 || block_threads > 1024 ||
      block_threads % 64 || !sink)
    return 1;
  // 32-bit unit indices: the last index plus kUnroll grid strides stays below 2^32
  if (rows > (uint64_t{1} << 32) ||
      rows * per + kUnroll * static_cast<uint64_t>(grid_blocks) * block_threads >= (uint64_t{1} << 32))
    return 1;
  if ((read_units && (!src || reinterpret_cast<uintptr_t>(src) % 16)) ||
      (write_units && (!dst || reinterpret_cast<uintptr_t>(dst) % 16)))
    return 1;
  if (layout != 0 && layout != 1) return 1;
  if (layout == 1) {
    // every kind needs a workgroup: at least one full group of read_units + write_units
    if (grid_blocks < per) return 1;
    hipLaunchKernelGGL(stream_probe_split_kernel, dim3(grid_blocks), dim3(block_threads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                       static_cast<uint32_t>(rows * read_units), static_cast<uint32_t>(rows * write_units),
                       read_units, write_units, key, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
  }
  const uint64_t m = ((uint64_t{1} << 32) + per - 1) / per;
  hipLaunchKernelGGL(stream_probe_kernel, dim3(grid_blocks), dim3(block_threads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), static_cast<uint32_t>(rows * per),
                     static_cast<uint32_t>(per), m, read_units, write_units, key, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
