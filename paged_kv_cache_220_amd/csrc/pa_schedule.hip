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
  __shared__ int scan[kMaxQueueBuckets];
  const int tid = threadIdx.x;
  const int P = a.partition_tokens;
  const int full = P / kTileTokens;             // bucket of a full partition
  const int hkv = a.num_kv_heads;
  const int qbs = a.q_blocks;
  const int units_per_seq = hkv * qbs;   // unit = (s * q_blocks + qb) * Hkv + kvh
  int2* items = const_cast<int2*>(a.queue_items);
  for (int b = tid; b <= full; b += kPlanThreads) cnt[b] = 0;
  __syncthreads();
  for (int s = tid; s < a.num_seqs; s += kPlanThreads) {
    const int L = clamp_len(a, s);
    const int nfull = L / P;
    const int rem = L - nfull * P;
    if (nfull > 0) atomicAdd(&cnt[full], nfull * units_per_seq);
    if (rem > 0 || L == 0) atomicAdd(&cnt[(rem + kTileTokens - 1) / kTileTokens], units_per_seq);
  }
  __syncthreads();
  // Bucket offsets, longest first: an exclusive prefix sum over ranks
  // r = full - b (Hillis-Steele in LDS; a serial loop over up to 129 buckets
  // in one thread cost several microseconds of dependent LDS round trips).
  const int v = tid <= full ? cnt[full - tid] : 0;
  if (tid <= full) scan[tid] = v;
  __syncthreads();
  for (int d = 1; d <= full; d <<= 1) {
    const int add = (tid <= full && tid >= d) ? scan[tid - d] : 0;
    __syncthreads();
    if (tid <= full) scan[tid] += add;
    __syncthreads();
  }
  if (tid <= full) cur[full - tid] = scan[tid] - v;
  if (tid == full) *const_cast<int*>(a.queue_len) = scan[tid];
  __syncthreads();
  // Each sequence reserves its items of a bucket as one run (one LDS atomic
  // per bucket it touches, not one per item) and fills the run in order.
  for (int s = tid; s < a.num_seqs; s += kPlanThreads) {
    const int L = clamp_len(a, s);
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
  }
}

}  // namespace

hipError_t launch_plan(const Args& a, hipStream_t stream) {
  if (a.partition_tokens / kTileTokens >= kMaxQueueBuckets) return hipErrorInvalidValue;
  plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
