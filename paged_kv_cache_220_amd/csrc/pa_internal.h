// Internal declarations shared by the host API and the kernels of the
// PagedAttention decode library (gfx950). Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_decode.h"

namespace pa {

// Everything a partition or reduce kernel needs, passed by value.
struct Args {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* tables;
  const int32_t* seq_lens;
  void* out;
  float* part_o;   // [S][Hkv][max_parts][G*q_len][D]   unnormalised partition outputs
  float* part_m;   // [S][Hkv][max_parts][G*q_len]      partition running max (log2 domain)
  float* part_l;   // [S][Hkv][max_parts][G*q_len]      partition running sum
  int64_t block_stride;   // elements per physical block: Hkv * D * block_size
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;     // block_tables row length
  int32_t partition_tokens;
  int32_t max_parts;
  int32_t max_tokens;     // min(max_parts * partition_tokens, max_blocks * block_size)
  int32_t num_blocks;     // physical blocks in each cache
  float score_scale;      // scale * k_scale * log2(e): scores live in the log2 domain
  float v_scale;
  int32_t q_len;          // query positions per sequence (1 = decode)
  // List schedule (null queue_items: dense grid). The plan kernel fills
  // queue_items[0 .. *queue_len) with (sequence * Hkv + kv head, partition),
  // longest first; workgroup i of queue_workgroups processes item i.
  const int2* queue_items;
  const int* queue_len;
  int32_t queue_workgroups;
  int32_t waves_per_item;   // matrix-core kernel: waves sharing one work item (1, 2, 4)
  int32_t q_blocks;         // work items per (sequence, KV head): query blocks of up to 64 (query
                            // position, head) pairs, or groups of waves_per_item blocks that share tiles
  const float* k_bscale;    // per-(block, KV head) scales [num_blocks][num_kv_heads], or null
  const float* v_bscale;
};

// Host-side launchers; each returns the hipError_t of the launch.
hipError_t launch_valu(const Args& a, int q_dtype, int kv_dtype, int head_dim, int group,
                       hipStream_t stream);
// ev_start / ev_stop (may be null): recorded by the partition kernel's own
// dispatch at the start and end of its execution.
hipError_t launch_mfma(const Args& a, int q_dtype, int kv_dtype, int head_dim, int group,
                       hipStream_t stream, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_reduce(const Args& a, int q_dtype, int head_dim, int group, hipStream_t stream);
hipError_t launch_plan(const Args& a, hipStream_t stream);

bool valu_supported(int q_dtype, int kv_dtype, int head_dim, int group);
bool mfma_supported(int q_dtype, int kv_dtype, int head_dim, int group, int block_size, int q_len);
bool mfma_waves_supported(int group, int q_len, int nw);
// Tile sharing: with more than one query block per KV head and nw > 1, the nw
// waves of a work item take one query block each and share every K/V tile.
bool mfma_share_tiles(int group, int q_len, int nw);
// Work items per (sequence, KV head) of the matrix-core kernel (Args::q_blocks).
int mfma_item_blocks(int group, int q_len, int nw);
// Waves per item the planner takes for tile sharing.
int mfma_share_default_waves(int group, int q_len, long long max_len, int kv_dtype);

constexpr int kBlockSize = 16;     // tokens per physical block handled by the kernels
constexpr int kTileTokens = 64;    // partition lengths are multiples of this
constexpr int kMergeHeadsMaxParts = 8;  // merge by KV head (all its query heads per workgroup) up to this many partitions
constexpr int kMaxColumnGroups = 4; // matrix-core kernel: up to 64 (query position, head) pairs per work item
// Tile sharing: column groups (16 pairs each) per wave, and the most waves per
// item. Two groups per wave run two waves per SIMD; four groups per wave (one
// wave per SIMD, up to 4 waves per item) measured 4-8 % slower.
constexpr int kShareGroups = 2;
constexpr int kShareMaxWaves = kShareGroups == 2 ? 8 : 4;
constexpr int kMaxQueryLen = 4096;  // query positions per sequence
constexpr int kMaxQueueBuckets = 129;  // queue schedule: partitions of at most 128 tiles
constexpr int kResidentWorkgroups = 2048;  // gfx950: 256 CUs x 8 one-wave workgroups (planning)

// Sequence length as the kernels use it. Lengths outside [0, max_tokens]
// break a documented precondition; clamping keeps every access inside the
// table, the caches and the workspace (the output is then unspecified).
__device__ __forceinline__ int clamp_len(const Args& a, int s) {
  return min(max(a.seq_lens[s], 0), a.max_tokens);
}

// Work item of a partition-kernel workgroup. The grid is
// (num_kv_heads * num_seqs, max_parts): consecutive workgroups differ in KV
// head and sequence, and the partition index is the slowest. The hardware
// deals workgroup i to XCD i % 8, so every partition index, and in particular
// partition 0 that each sequence has, is spread over all eight XCDs whatever
// the head count or length mix. Partitions are dispatched last index first:
// the deep partitions that only long sequences have start early, and the
// first partitions, which include every short sequence, fill the tail.
struct Item {
  int kvh, qb, s, part;
};
// blockIdx.x = kvh + Hkv * (qb + q_blocks * s): the query blocks of one
// (sequence, KV head) are Hkv workgroups apart, so with Hkv a multiple of the
// 8 XCDs they share an XCD (and its L2 for the K/V tiles they all read) and
// are dispatched close together.
__device__ __forceinline__ Item work_item(const Args& a) {
  Item it;
  const int per_seq = a.num_kv_heads * a.q_blocks;
  it.s = blockIdx.x / per_seq;
  const int r = blockIdx.x - it.s * per_seq;
  it.qb = r / a.num_kv_heads;
  it.kvh = r - it.qb * a.num_kv_heads;
  it.part = a.max_parts - 1 - (int)blockIdx.y;
  return it;
}
__host__ __forceinline__ dim3 partition_grid(const Args& a) {
  return dim3((unsigned)a.num_kv_heads * (unsigned)a.q_blocks * (unsigned)a.num_seqs, (unsigned)a.max_parts, 1);
}

// Physical block id, clamped into the pool for the same reason.
__device__ __forceinline__ int64_t clamp_block(const Args& a, int32_t id) {
  return (int64_t)min(max(id, 0), a.num_blocks - 1);
}

}  // namespace pa
