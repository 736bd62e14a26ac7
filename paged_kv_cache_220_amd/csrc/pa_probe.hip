// Streaming-read probe (gfx950): reads a buffer once with 128-bit
// non-temporal loads and folds it into XOR checksums (one word per
// workgroup), nothing else. Its
// rate is the practical read ceiling the decode kernels are compared with.
//
// Each workgroup reads contiguous 32 KiB chunks (kUnroll loads per thread,
// all in flight before any is used; one load instruction of the workgroup
// covers 4 KiB), and the chunks are dealt round-robin over a grid of up to
// 4096 workgroups. Measured on MI355X against other shapes of the same
// kernel: one wave per contiguous chunk reached 6.7-6.9 TB/s, loads strided
// a whole grid apart 5.8-6.5 TB/s, cached instead of non-temporal loads
// 0.6-0.9 TB/s less; this one 7.0 TB/s. (With one atomic XOR per wave into
// a single word instead of a store per workgroup, the contended atomics at
// the end of the pass cost about 90 us of a 4 GiB read.)

#include <hip/hip_runtime.h>

#include "pa_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kChunk = kThreads * kUnroll;     // 16-byte elements per workgroup chunk (32 KiB)
constexpr int kMaxWorkgroups = PA_PROBE_SINK_WORDS;
static_assert(kChunk * 16 == PA_PROBE_CHUNK_BYTES, "chunk size as declared");

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                               uint32_t* sink) {
  const int64_t step = (int64_t)gridDim.x * kChunk;
  uint32_t acc = 0;
  int64_t c = (int64_t)blockIdx.x * kChunk;
  for (; c + kChunk <= n16; c += step) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + c + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the last, partial chunk (at most one workgroup reaches here with c < n16)
  for (int64_t i = c + threadIdx.x; i < n16; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup: a plain store, no contended atomics
  __shared__ uint32_t wave_acc[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) wave_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) w ^= wave_acc[i];
    sink[blockIdx.x] = w;
  }
}

}  // namespace

extern "C" int pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return PA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return PA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return PA_ERR_ALIGN;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t want = (n16 + kChunk - 1) / kChunk;
  const int grid = (int)(want < kMaxWorkgroups ? want : kMaxWorkgroups);
  read_probe_kernel<<<grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
