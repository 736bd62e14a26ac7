// Work list for the list schedule of the partition kernel (gfx950).
//
// With a skewed length mix the dense (KV head, sequence, partition) grid is
// mostly empty workgroups, and the few long partitions dispatched late leave a
// tail in which most CUs idle. This kernel (one workgroup) lists the items that
// exist, ordered by their number of 64-token tiles, longest first (a counting
// sort: full partitions, then each sequence's last partial partition by
// length, then empty sequences, which still get a zero output row). The
// partition kernel's workgroup i then takes item i, so long items start first
// and the short ones fill the end. It also writes the list length the
// partition kernel reads, so nothing else needs clearing first.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const Args a) {
  __shared__ int cnt[kMaxQueueBuckets];
  __shared__ int cur[kMaxQueueBuckets];
  const int tid = threadIdx.x;
  const int P = a.partition_tokens;
  const int full = P / kTileTokens;             // bucket of a full partition
  const int hkv = a.num_kv_heads;
  const int qbs = a.q_blocks;
  const int units_per_seq = hkv * qbs;   // unit = (s * q_blocks + qb) * Hkv + kvh
  int2* items = const_cast<int2*>(a.queue_items);
  for (int b = tid; b <= full; b += kPlanThreads) cnt[b] = 0;
  // The lengths of this thread's first kKeep sequences stay in registers
  // for the second pass (one read of seq_lens for up to kKeep * 1024).
  constexpr int kKeep = 4;
  int keep[kKeep];
  __syncthreads();
  auto count = [&](int L) {
    const int nfull = L / P;
    const int rem = L - nfull * P;
    if (nfull > 0) atomicAdd(&cnt[full], nfull * units_per_seq);
    if (rem > 0 || L == 0) atomicAdd(&cnt[(rem + kTileTokens - 1) / kTileTokens], units_per_seq);
  };
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    const int s = tid + k * kPlanThreads;
    keep[k] = s < a.num_seqs ? clamp_len(a, s) : 0;
    if (s < a.num_seqs) count(keep[k]);
  }
  for (int s = tid + kKeep * kPlanThreads; s < a.num_seqs; s += kPlanThreads) count(clamp_len(a, s));
  __syncthreads();
  // Bucket offsets, longest first: an exclusive prefix sum over ranks
  // r = full - b, taken by the first wave alone (up to 129 buckets, three
  // per lane, then a shuffle scan over the lane totals), so only two
  // workgroup barriers remain around it.
  if (tid < 64) {
    int v[3], run = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int r = 3 * tid + k;
      v[k] = r <= full ? cnt[full - r] : 0;
      run += v[k];
    }
    int incl = run;   // inclusive scan of the lane totals
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d, 64);
      if (tid >= d) incl += up;
    }
    int off = incl - run;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int r = 3 * tid + k;
      if (r <= full) cur[full - r] = off;
      off += v[k];
    }
    if (tid == 63) *const_cast<int*>(a.queue_len) = incl;
  }
  __syncthreads();
  // Each sequence reserves its items of a bucket as one run (one LDS atomic
  // per bucket it touches, not one per item) and fills the run in order.
  auto fill = [&](int s, int L) {
    const int nfull = L / P;
    const int rem = L - nfull * P;
    if (nfull > 0) {
      int2* run = items + atomicAdd(&cur[full], nfull * units_per_seq);
      for (int u = 0; u < units_per_seq; ++u)
        for (int p = 0; p < nfull; ++p) run[u * nfull + p] = make_int2(s * units_per_seq + u, p);
    }
    if (rem > 0 || L == 0) {
      int2* run = items + atomicAdd(&cur[(rem + kTileTokens - 1) / kTileTokens], units_per_seq);
      for (int u = 0; u < units_per_seq; ++u) run[u] = make_int2(s * units_per_seq + u, nfull);
    }
  };
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    const int s = tid + k * kPlanThreads;
    if (s < a.num_seqs) fill(s, keep[k]);
  }
  for (int s = tid + kKeep * kPlanThreads; s < a.num_seqs; s += kPlanThreads) fill(s, clamp_len(a, s));
}

}  // namespace

hipError_t launch_plan(const Args& a, hipStream_t stream) {
  static_assert(kMaxQueueBuckets <= 3 * 64, "the bucket scan takes three buckets per lane of one wave");
  if (a.partition_tokens / kTileTokens >= kMaxQueueBuckets) return hipErrorInvalidValue;
  plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
