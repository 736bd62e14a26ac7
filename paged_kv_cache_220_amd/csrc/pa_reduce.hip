// Merge of per-partition softmax states into the decode output (gfx950).
//
// A sequence longer than one context partition leaves, per partition p and
// query head, its running max m_p (log2 domain), running sum l_p and
// unnormalised output o_p. They combine with the same rescaling the
// online-softmax update of the PagedAttention kernel pseudocode (vLLM page)
// applies between blocks:
//   M = max_p m_p,  l = sum_p 2^(m_p - M) l_p,  out = sum_p 2^(m_p - M) o_p / l.
// Sequences with a single partition were written directly by the partition
// kernel and are skipped here.
//
// One workgroup per (sequence, query head); one thread per output element.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <int QDT>
__global__ __launch_bounds__(128) void reduce_kernel(const Args a, int head_dim, int group) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int L = clamp_len(a, s);
  const int P = a.partition_tokens;
  const int nparts = (L + P - 1) / P;
  if (nparts <= 1) return;
  const int kvh = h / group;
  const int g = h - kvh * group;
  const int64_t item0 = ((int64_t)s * a.num_kv_heads + kvh) * a.max_parts;

  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.part_m[(item0 + p) * group + g]);

  for (int d = threadIdx.x; d < head_dim; d += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int p = 0; p < nparts; ++p) {
      const int64_t it = (item0 + p) * group + g;
      const float w = exp2f(a.part_m[it] - M);
      den = fmaf(w, a.part_l[it], den);
      num = fmaf(w, a.part_o[it * head_dim + d], num);
    }
    store_out<QDT>(a.out, ((int64_t)s * a.num_heads + h) * head_dim + d, num / den);
  }
}

}  // namespace

hipError_t launch_reduce(const Args& a, int q_dtype, int head_dim, int group, hipStream_t stream) {
  const dim3 grid(a.num_heads, a.num_seqs);
  const int threads = head_dim >= 128 ? 128 : 64;
  if (q_dtype == kF32) {
    reduce_kernel<kF32><<<grid, threads, 0, stream>>>(a, head_dim, group);
  } else if (q_dtype == kBF16) {
    reduce_kernel<kBF16><<<grid, threads, 0, stream>>>(a, head_dim, group);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
