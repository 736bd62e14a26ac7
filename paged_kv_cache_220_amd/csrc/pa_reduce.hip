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
// With several query positions per sequence, (query position, head) pairs are
// merged alike; a query whose window holds no token in any partition gets a
// zero row.
//
// Up to 8 partitions per sequence (the usual case: partitions are made as
// long as the grid allows): one workgroup of 256 threads per (sequence, KV
// head, 8 of its query heads), 8 heads x 32 column groups of 4 output
// elements. Each thread issues the 128-bit loads of o_p for all partitions
// at once (a wave reads 512 contiguous bytes per partition and head) and
// combines them in partition order. One workgroup per KV head instead of one
// per query head means 8x fewer workgroups at G = 8, most of them empty when
// most sequences fit one partition.
//
// More partitions: one workgroup per (sequence, query head), 8 partition
// groups x 32 column groups. Each thread walks every 8th partition, folding
// them into a running (m, l, o) by the same rule, so all loads go out in one
// round trip; the 8 group states then meet in LDS in a fixed order.
//
// Both orders give the same result for up to 8 partitions (a group that
// holds one partition keeps its state unchanged), and neither depends on
// timing.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = 8;          // partition groups
constexpr int kCols = 32;           // column groups of 4 elements: head_dim <= 128

template <int QDT>
__global__ __launch_bounds__(kThreads) void reduce_kernel(const Args a, int head_dim, int group) {
  const int qi = blockIdx.x / a.num_heads;          // query position (0 for decode)
  const int h = blockIdx.x - qi * a.num_heads;
  const int s = blockIdx.y;
  const int L = clamp_len(a, s);
  const int P = a.partition_tokens;
  const int nparts = (L + P - 1) / P;
  if (nparts <= 1) return;
  const int kvh = h / group;
  const int GV = group * a.q_len;                     // virtual heads (query position, head) per KV head
  const int g = qi * group + (h - kvh * group);
  const int64_t item0 = ((int64_t)s * a.num_kv_heads + kvh) * a.max_parts;
  const int64_t orow = (((int64_t)s * a.q_len + qi) * a.num_heads + h) * head_dim;
  const int tid = threadIdx.x;

  __shared__ float red_m[kGroups];
  __shared__ float red_l[kGroups];
  __shared__ float red_o[kGroups][kCols * 4];

  const int pg = tid / kCols;
  const int col = (tid % kCols) * 4;
  const bool active = col < head_dim;
  // Running state of this partition group. A group that has seen no token
  // keeps m = -inf; subtracting 0 instead then gives weights 2^-inf = 0.
  float m = -INFINITY, l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
  for (int p = pg; p < nparts; p += kGroups) {
    const int64_t it = (item0 + p) * GV + g;
    const float mp = a.part_m[it];
    const float lp = a.part_l[it];
    const float4 op = active ? *reinterpret_cast<const float4*>(a.part_o + it * head_dim + col)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    const float mn = fmaxf(m, mp);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float sa = exp2f(m - mu), sb = exp2f(mp - mu);
    l = l * sa + lp * sb;
    o.x = o.x * sa + op.x * sb;
    o.y = o.y * sa + op.y * sb;
    o.z = o.z * sa + op.z * sb;
    o.w = o.w * sa + op.w * sb;
    m = mn;
  }
  if (active) {
    red_o[pg][col + 0] = o.x;
    red_o[pg][col + 1] = o.y;
    red_o[pg][col + 2] = o.z;
    red_o[pg][col + 3] = o.w;
  }
  if (tid % kCols == 0) {
    red_m[pg] = m;
    red_l[pg] = l;
  }
  __syncthreads();

  if (tid < head_dim) {
    float M = red_m[0];
#pragma unroll
    for (int k = 1; k < kGroups; ++k) M = fmaxf(M, red_m[k]);
    if (M == -INFINITY) {
      // no partition saw a token this query may attend (query window longer than the sequence)
      store_out<QDT>(a.out, orow + tid, 0.f);
      return;
    }
    float acc = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
      const float w = exp2f(red_m[k] - M);
      acc += red_o[k][tid] * w;
      den += red_l[k] * w;
    }
    store_out<QDT>(a.out, orow + tid, acc / den);
  }
}

// Up to kGroups partitions: partition p's state is loaded for every p <
// kGroups (index clamped to the last partition, so every load is in bounds
// and issues without a branch) and the states past nparts are given weight 0.
template <int QDT>
__global__ __launch_bounds__(kThreads) void reduce_heads_kernel(const Args a, int head_dim, int group) {
  const int GV = group * a.q_len;                     // virtual heads (query position, head) per KV head
  const int chunks = (GV + kGroups - 1) / kGroups;
  const int kvh = blockIdx.x / chunks;
  const int g = (blockIdx.x - kvh * chunks) * kGroups + threadIdx.x / kCols;
  const int s = blockIdx.y;
  const int L = clamp_len(a, s);
  const int P = a.partition_tokens;
  const int nparts = (L + P - 1) / P;
  if (nparts <= 1) return;
  const int col = (threadIdx.x % kCols) * 4;
  if (g >= GV || col >= head_dim) return;
  const int qi = g / group;
  const int h = kvh * group + (g - qi * group);
  const int64_t item0 = ((int64_t)s * a.num_kv_heads + kvh) * a.max_parts;
  const int64_t orow = (((int64_t)s * a.q_len + qi) * a.num_heads + h) * head_dim;

  float mp[kGroups], lp[kGroups];
  float4 op[kGroups];
#pragma unroll
  for (int p = 0; p < kGroups; ++p) {
    const int64_t it = (item0 + min(p, nparts - 1)) * GV + g;
    mp[p] = a.part_m[it];
    lp[p] = a.part_l[it];
    op[p] = *reinterpret_cast<const float4*>(a.part_o + it * head_dim + col);
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kGroups; ++p)
    if (p < nparts) M = fmaxf(M, mp[p]);
  if (M == -INFINITY) {
    // no partition saw a token this query may attend (query window longer than the sequence)
#pragma unroll
    for (int j = 0; j < 4; ++j) store_out<QDT>(a.out, orow + col + j, 0.f);
    return;
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
#pragma unroll
  for (int p = 0; p < kGroups; ++p) {
    const float w = p < nparts ? exp2f(mp[p] - M) : 0.f;
    acc.x += op[p].x * w;
    acc.y += op[p].y * w;
    acc.z += op[p].z * w;
    acc.w += op[p].w * w;
    den += lp[p] * w;
  }
  store_out<QDT>(a.out, orow + col + 0, acc.x / den);
  store_out<QDT>(a.out, orow + col + 1, acc.y / den);
  store_out<QDT>(a.out, orow + col + 2, acc.z / den);
  store_out<QDT>(a.out, orow + col + 3, acc.w / den);
}

}  // namespace

hipError_t launch_reduce(const Args& a, int q_dtype, int head_dim, int group, hipStream_t stream) {
  if (head_dim > kCols * 4 || head_dim % 4 != 0) return hipErrorInvalidValue;
  static_assert(kMergeHeadsMaxParts == kGroups, "the head-wise merge loads one state per partition group");
  if (a.max_parts <= kMergeHeadsMaxParts) {
    const int gv = group * a.q_len;
    const dim3 grid(a.num_kv_heads * ((gv + kGroups - 1) / kGroups), a.num_seqs);
    if (q_dtype == kF32) {
      reduce_heads_kernel<kF32><<<grid, kThreads, 0, stream>>>(a, head_dim, group);
    } else if (q_dtype == kBF16) {
      reduce_heads_kernel<kBF16><<<grid, kThreads, 0, stream>>>(a, head_dim, group);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid(a.num_heads * a.q_len, a.num_seqs);
  if (q_dtype == kF32) {
    reduce_kernel<kF32><<<grid, kThreads, 0, stream>>>(a, head_dim, group);
  } else if (q_dtype == kBF16) {
    reduce_kernel<kBF16><<<grid, kThreads, 0, stream>>>(a, head_dim, group);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
