// stream_read.hip -- the streaming-read ceiling the verify is measured against
// (a measurement kernel of the benchmark, not part of the verify).
//
// Reads `bytes` from `base` once, one 16 KiB chunk per workgroup of 256
// threads, four non-temporal 128-bit loads per thread (each wave instruction
// covers 1 KiB contiguous), the same access pattern as the verify's
// producers, and writes one XOR word per workgroup so that no load is dropped.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svs {

constexpr int WG = 256;
constexpr int CHUNK_BYTES = 16384;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(WG) void k_stream_read(const unsigned char* __restrict__ base,
                                                    size_t bytes, unsigned int* __restrict__ out) {
  const size_t c0 = (size_t)blockIdx.x * CHUNK_BYTES;
  unsigned int x = 0;
#pragma unroll
  for (int i = 0; i < CHUNK_BYTES / (WG * 16); ++i) {
    const size_t off = c0 + ((size_t)i * WG + threadIdx.x) * 16;
    if (off + 16 <= bytes) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  // one word per workgroup: lanes combined through LDS
  __shared__ unsigned int red[WG];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int s = WG / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace svs

extern "C" {

// Number of output words (workgroups) a read of `bytes` writes.
size_t sv_stream_read_words(size_t bytes) {
  return (bytes + svs::CHUNK_BYTES - 1) / svs::CHUNK_BYTES;
}

// Enqueue one streaming read of `bytes` bytes at `base` (16-byte aligned) on
// `stream`; `out` holds sv_stream_read_words(bytes) words.  0 on success.
int sv_stream_read(const void* base, size_t bytes, unsigned int* out, void* stream) {
  if (!base || !out || bytes == 0 || ((uintptr_t)base & 15) != 0) return 1;
  const size_t g = sv_stream_read_words(bytes);
  if (g >= (1ull << 31)) return 2;
  hipLaunchKernelGGL(svs::k_stream_read, dim3((unsigned)g), dim3(svs::WG), 0, (hipStream_t)stream,
                     (const unsigned char*)base, bytes, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
