// C ABI of the PagedAttention decode library: argument validation, launch
// planning (context partitions, workspace layout) and kernel launches.
// Validation runs entirely on the host before any HIP call.

#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "pa_internal.h"

namespace {

using pa::Args;

constexpr int kVersionMajor = 0;
constexpr int kVersionMinor = 1;
constexpr size_t kAlign = 256;
constexpr int kMaxParts = 65535;   // partitions per sequence: the grid's y dimension

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Plan {
  int kernel = PA_KERNEL_VALU;
  int group = 1;
  int q_len = 1;
  int q_blocks = 1;   // blocks of up to 64 (query position, head) pairs per KV head
  int max_len = 0;
  int partition_tokens = 0;
  int max_parts = 1;
  int schedule = PA_SCHEDULE_GRID;
  int waves_per_item = 1;
  size_t off_m = 0, off_l = 0, off_items = 0, off_qlen = 0, ws_bytes = 0;
  long long grid = 0, reduce_grid = 0;
};

int q_len_of(const pa_dims_t* d) { return d->q_len > 1 ? d->q_len : 1; }

int check_dims(const pa_dims_t* d, int32_t hkv) {
  if (d == nullptr) return PA_ERR_NULL;
  if (d->num_seqs <= 0 || d->num_heads <= 0 || d->head_dim <= 0 || d->num_blocks <= 0 ||
      d->block_size <= 0 || d->max_blocks_per_seq <= 0 || hkv <= 0)
    return PA_ERR_SHAPE;
  if (d->num_heads % hkv != 0) return PA_ERR_SHAPE;
  if (d->max_seq_len < 0 || d->partition_tokens < 0) return PA_ERR_SHAPE;
  if ((long long)d->max_seq_len > (long long)d->max_blocks_per_seq * d->block_size) return PA_ERR_SHAPE;
  if (d->partition_tokens % pa::kTileTokens != 0) return PA_ERR_SHAPE;
  if (!isfinite(d->k_scale) || !isfinite(d->v_scale)) return PA_ERR_SHAPE;
  if (!(d->k_scale > 0.f)) return PA_ERR_SHAPE;   // scores scale by a positive factor
  if (d->q_len < 0) return PA_ERR_SHAPE;
  // per-block scales: both or neither; required for int4, allowed for fp8
  const bool fp8 = d->kv_dtype == PA_DTYPE_FP8_E5M2 || d->kv_dtype == PA_DTYPE_FP8_E4M3;
  if ((d->k_block_scales == nullptr) != (d->v_block_scales == nullptr)) return PA_ERR_NULL;
  if (d->kv_dtype == PA_DTYPE_INT4 && d->k_block_scales == nullptr) return PA_ERR_NULL;
  if (d->k_block_scales != nullptr && d->kv_dtype != PA_DTYPE_INT4 && !fp8) return PA_ERR_UNSUPPORTED;
  if (!aligned(d->k_block_scales, 4) || !aligned(d->v_block_scales, 4)) return PA_ERR_ALIGN;
  if (d->kernel < PA_KERNEL_AUTO || d->kernel > PA_KERNEL_MFMA) return PA_ERR_UNSUPPORTED;
  if (d->schedule < PA_SCHEDULE_AUTO || d->schedule > PA_SCHEDULE_QUEUE) return PA_ERR_UNSUPPORTED;
  if (d->waves_per_item < 0 || d->waves_per_item > 8 || d->waves_per_item == 5 || d->waves_per_item == 6 ||
      d->waves_per_item == 7)
    return PA_ERR_UNSUPPORTED;
  if (d->block_size != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  const int group = d->num_heads / hkv;
  const int ql = q_len_of(d);
  const long long qblocks = ((long long)group * ql + 63) / 64;
  if ((long long)d->num_seqs * hkv * qblocks > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;  // grid x limit
  if ((long long)d->num_heads * ql > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;   // merge grid x
  const bool valu_ok = ql == 1 && d->k_block_scales == nullptr &&
                       pa::valu_supported(d->q_dtype, d->kv_dtype, d->head_dim, group);
  const bool mfma_ok = pa::mfma_supported(d->q_dtype, d->kv_dtype, d->head_dim, group, d->block_size, ql);
  if (d->kernel == PA_KERNEL_VALU && !valu_ok) return PA_ERR_UNSUPPORTED;
  if (d->kernel == PA_KERNEL_MFMA && !mfma_ok) return PA_ERR_UNSUPPORTED;
  if (!valu_ok && !mfma_ok) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int make_plan(const pa_dims_t* d, int32_t hkv, Plan* p) {
  const int st = check_dims(d, hkv);
  if (st != PA_OK) return st;
  p->group = d->num_heads / hkv;
  p->q_len = q_len_of(d);
  if (d->kernel == PA_KERNEL_AUTO) {
    p->kernel = pa::mfma_supported(d->q_dtype, d->kv_dtype, d->head_dim, p->group, d->block_size, p->q_len)
                    ? PA_KERNEL_MFMA
                    : PA_KERNEL_VALU;   // check_dims guarantees the vector kernel takes what the other does not
  } else {
    p->kernel = d->kernel;
  }
  p->max_len = d->max_seq_len > 0 ? d->max_seq_len : d->max_blocks_per_seq * d->block_size;
  // Query blocks (up to 64 (query position, head) pairs each). With more than
  // one, the matrix-core kernel by default gives an item 2, 4 or (past 4096
  // tokens) 8 waves of 32 pairs each, and the waves share every K/V tile;
  // waves_per_item = 1 keeps one block of 64 per item.
  const int gv = p->group * p->q_len;   // (query position, head) pairs per KV head
  const int ncg = gv <= 16 ? 1 : gv <= 32 ? 2 : 4;
  const int blocks64 = (gv + 16 * pa::kMaxColumnGroups - 1) / (16 * pa::kMaxColumnGroups);
  const bool mfma = p->kernel == PA_KERNEL_MFMA;
  int share_nw = 0;   // waves per item when they share tiles
  if (mfma && blocks64 > 1 && d->waves_per_item != 1) {
    share_nw = d->waves_per_item > 0 ? d->waves_per_item
                                        : pa::mfma_share_default_waves(p->group, p->q_len, p->max_len, d->kv_dtype);
    if (!pa::mfma_share_tiles(p->group, p->q_len, share_nw) || share_nw > pa::kShareMaxWaves)
      return PA_ERR_UNSUPPORTED;
  }
  p->q_blocks = mfma ? pa::mfma_item_blocks(p->group, p->q_len, share_nw > 0 ? share_nw : 1) : 1;
  // Every wave keeps about one 64-token tile of K and V in flight. Covering
  // HBM latency at full bandwidth takes about as many waves as the chip holds
  // at once: 2048 (two waves per SIMD), and 3072 with int4 tiles (8 KiB; that
  // kernel stages K in LDS and runs three waves per SIMD). The fp8 kernel can
  // hold three as well, but with its K copies and V loads overlapping the
  // compute two waves per SIMD measured 1-2 % faster (fp8 batches of 32K and
  // of shared-prefix sequences). Partitions are
  // made as long as possible (up to 4096 tokens, 8192 with tile sharing:
  // start-up and merge traffic are amortised) and the waves come from
  // splitting each item over 1 to 4 waves; partitions are shortened only when
  // even 4 waves per item would not reach the target.
  const long long units = (long long)d->num_seqs * hkv * (p->kernel == PA_KERNEL_MFMA ? p->q_blocks : 1);
  // three waves per SIMD: int4. The tile-sharing kernels run two waves per
  // SIMD (2048 on the chip).
  const bool three_waves = d->kv_dtype == PA_DTYPE_INT4;
  const long long target_waves = share_nw > 0 ? 2048 : three_waves ? 3072 : 2048;
  const int max_item_waves = share_nw > 0 ? share_nw : 4;
  auto items_for = [&](long long P) { return units * ((p->max_len + P - 1) / P); };
  int P = d->partition_tokens;
  if (P == 0) {
    // Tile-sharing items run up to 8192 tokens: with every item resident at
    // once, half the partitions halve the merge traffic of their (larger)
    // states and the per-item start-up (measured 3-4 % per call at 16 to 64
    // positions over 32K tokens); decode stays at 4096.
    long long cap = share_nw > 0 ? 8192 : 4096;
    while (cap / 2 >= p->max_len && cap > pa::kTileTokens) cap /= 2;   // no longer than the longest sequence needs
    P = (int)cap;
    while (P > 256 && items_for(P) * max_item_waves < target_waves) P /= 2;
  }
  if (d->partition_tokens == 0) {
    while ((p->max_len + (long long)P - 1) / P > kMaxParts) P *= 2;   // grid y limit
  }
  p->partition_tokens = P;
  p->max_parts = p->max_len > 0 ? (int)((p->max_len + (long long)P - 1) / P) : 1;
  if (p->max_parts < 1) p->max_parts = 1;
  if (p->max_parts > kMaxParts) return PA_ERR_UNSUPPORTED;
  p->grid = (long long)p->max_parts * hkv * p->q_blocks * d->num_seqs;
  // merge: one workgroup per (sequence, KV head, 8 virtual heads) up to 8
  // partitions, else one per (sequence, virtual head)
  const long long gv_all = (long long)p->group * p->q_len;
  p->reduce_grid = p->max_parts <= 1 ? 0
                   : p->max_parts <= pa::kMergeHeadsMaxParts ? (long long)hkv * ((gv_all + 7) / 8) * d->num_seqs
                                                             : (long long)d->num_heads * p->q_len * d->num_seqs;
  // List schedule: for the matrix-core kernel when asked, or when the dense
  // grid is far larger than the resident workgroups (a skewed or sparse
  // length mix leaves most of it empty and its long partitions in the tail).
  const bool queue_ok = p->kernel == PA_KERNEL_MFMA && P / pa::kTileTokens < pa::kMaxQueueBuckets;
  if (d->schedule == PA_SCHEDULE_QUEUE) {
    if (!queue_ok) return PA_ERR_UNSUPPORTED;
    p->schedule = PA_SCHEDULE_QUEUE;
  } else if (d->schedule == PA_SCHEDULE_AUTO && queue_ok && p->grid > 4LL * pa::kResidentWorkgroups) {
    p->schedule = PA_SCHEDULE_QUEUE;
  } else {
    p->schedule = PA_SCHEDULE_GRID;
  }
  // Waves per item (matrix-core kernel): the list schedule splits its long
  // items four ways so the tail is short; the grid splits items while the
  // grid still fits the wave target, keeping at least 4 tiles per wave.
  if (p->kernel != PA_KERNEL_MFMA) {
    if (d->waves_per_item > 1) return PA_ERR_UNSUPPORTED;
    p->waves_per_item = 1;
  } else if (share_nw > 0) {
    p->waves_per_item = share_nw;
  } else if (d->waves_per_item > 0) {
    if (!pa::mfma_waves_supported(p->group, p->q_len, d->waves_per_item)) return PA_ERR_UNSUPPORTED;
    p->waves_per_item = d->waves_per_item;
  } else if (p->schedule == PA_SCHEDULE_QUEUE) {
    p->waves_per_item = ncg == 1 ? 4 : 2;
  } else {
    const long long tiles = (std::min<long long>(P, p->max_len) + pa::kTileTokens - 1) / pa::kTileTokens;
    // the most waves (1 to 4) for which the grid fits the target and every
    // wave keeps at least 4 tiles: 3 fills the three waves per SIMD of the
    // int4 kernel when the grid is a third of them. With fp8 and whole
    // sequences as items (one partition) a wave keeps at least 8: on the chat
    // batch (at most 8 tiles) one wave per item ran 6-7 % faster than two,
    // where bf16 ties and int4 prefers two.
    const bool fp8 = d->kv_dtype == PA_DTYPE_FP8_E5M2 || d->kv_dtype == PA_DTYPE_FP8_E4M3;
    const long long min_tiles = fp8 && p->max_parts == 1 ? 8 : 4;
    int nw = 1;
    for (int w = 2; w <= 4; ++w)
      if (p->grid * w <= target_waves && tiles >= min_tiles * w && pa::mfma_waves_supported(p->group, p->q_len, w))
        nw = w;
    p->waves_per_item = nw;
  }
  size_t off = 0;
  if (p->max_parts > 1) {
    const size_t items = (size_t)d->num_seqs * hkv * p->max_parts * p->group * p->q_len;
    const size_t o_bytes = items * d->head_dim * sizeof(float);
    p->off_m = align_up(o_bytes, kAlign);
    p->off_l = p->off_m + align_up(items * sizeof(float), kAlign);
    off = p->off_l + align_up(items * sizeof(float), kAlign);
  }
  if (p->schedule == PA_SCHEDULE_QUEUE) {
    p->off_items = off;
    p->off_qlen = off + align_up((size_t)p->grid * sizeof(int2), kAlign);
    off = p->off_qlen + kAlign;          // list length
  }
  p->ws_bytes = off;
  return PA_OK;
}

// Every host-side check of a decode call (pointers, sizes, plan, scale,
// alignment); the entry points run it before any HIP call.
int validate(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
             const int32_t* seq_lens, int32_t hkv, float scale, void* out, const pa_dims_t* dims, Plan* p) {
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return PA_ERR_NULL;
  const int st = make_plan(dims, hkv, p);
  if (st != PA_OK) return st;
  if (!isfinite(scale) || !(scale > 0.f) || !isfinite(scale * dims->k_scale * 1.4426950408889634f))
    return PA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return PA_ERR_ALIGN;
  return PA_OK;
}

int run(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
        const int32_t* seq_lens, int32_t hkv, float scale, void* out, const pa_dims_t* dims,
        void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
        hipEvent_t ev2) {
  Plan p;
  const int st = validate(q, k_cache, v_cache, block_tables, seq_lens, hkv, scale, out, dims, &p);
  if (st != PA_OK) return st;
  if (p.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < p.ws_bytes || !aligned(workspace, kAlign)))
    return PA_ERR_WORKSPACE;

  Args a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.part_o = p.max_parts > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_m = p.max_parts > 1 ? reinterpret_cast<float*>(ws + p.off_m) : nullptr;
  a.part_l = p.max_parts > 1 ? reinterpret_cast<float*>(ws + p.off_l) : nullptr;
  a.block_stride = (int64_t)hkv * dims->head_dim * dims->block_size;
  a.num_seqs = dims->num_seqs;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = hkv;
  a.max_blocks = dims->max_blocks_per_seq;
  a.partition_tokens = p.partition_tokens;
  a.max_parts = p.max_parts;
  {
    const long long cap_parts = (long long)p.max_parts * p.partition_tokens;
    const long long cap_table = (long long)dims->max_blocks_per_seq * dims->block_size;
    const long long cap = cap_parts < cap_table ? cap_parts : cap_table;
    a.max_tokens = (int32_t)(cap < 0x7fffffffLL ? cap : 0x7fffffffLL);
  }
  a.num_blocks = dims->num_blocks;
  a.score_scale = scale * dims->k_scale * 1.4426950408889634f;
  a.v_scale = dims->v_scale;
  a.q_len = p.q_len;
  a.q_blocks = p.q_blocks;
  a.k_bscale = dims->k_block_scales;
  a.v_bscale = dims->v_block_scales;
  a.queue_items = nullptr;
  a.queue_len = nullptr;
  a.queue_workgroups = 0;
  if (p.schedule == PA_SCHEDULE_QUEUE) {
    a.queue_items = reinterpret_cast<const int2*>(ws + p.off_items);
    a.queue_len = reinterpret_cast<const int*>(ws + p.off_qlen);
    a.queue_workgroups = (int32_t)p.grid;            // the list never holds more items than the dense grid
  }
  a.waves_per_item = p.waves_per_item;

  // Timing: the matrix-core kernel's dispatch records ev0 / ev1 itself at the
  // start and end of its execution (no extra stream markers, whose cost would
  // land in every timed step); around the vector kernel they are recorded on
  // the stream. The work-list plan kernel, when it runs, precedes ev0.
  const bool mfma = p.kernel == PA_KERNEL_MFMA;
  if (p.schedule == PA_SCHEDULE_QUEUE && pa::launch_plan(a, stream) != hipSuccess) return PA_ERR_HIP;
  if (!mfma && ev0 && hipEventRecord(ev0, stream) != hipSuccess) return PA_ERR_HIP;
  hipError_t e = mfma ? pa::launch_mfma(a, dims->q_dtype, dims->kv_dtype, dims->head_dim, p.group, stream, ev0, ev1)
                      : pa::launch_valu(a, dims->q_dtype, dims->kv_dtype, dims->head_dim, p.group, stream);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (!mfma && ev1 && hipEventRecord(ev1, stream) != hipSuccess) return PA_ERR_HIP;
  if (p.max_parts > 1) {
    e = pa::launch_reduce(a, dims->q_dtype, dims->head_dim, p.group, stream);
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  if (ev2 && hipEventRecord(ev2, stream) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

// Scratch of pa_decode_noalloc: a device array of fixed size in this
// library's code object, one copy per GPU (each device that loads the code
// object holds its own), kept until the process ends. In host code the name
// `scratch` is only a stand-in: its device address on a GPU comes from
// hipGetSymbolAddress with that GPU current, looked up once per device and
// kept in scratch_ptr. Nothing in it has to start at zero: the partition
// kernel writes every state the merge kernel reads, and the plan kernel of the
// list schedule writes the list and its length.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU that runs `stream` (the current
// device for the null stream).
int scratch_for(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return PA_ERR_HIP;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return PA_ERR_HIP;
    dev = d;
  }
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return PA_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return PA_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return PA_ERR_HIP;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_workspace_bytes(const pa_dims_t* dims, int32_t num_kv_heads, int* status) {
  Plan p;
  const int st = make_plan(dims, num_kv_heads, &p);
  if (status) *status = st;
  return st == PA_OK ? p.ws_bytes : 0;
}

int pa_decode_plan(const pa_dims_t* dims, int32_t num_kv_heads, pa_plan_t* plan) {
  if (plan == nullptr) return PA_ERR_NULL;
  Plan p;
  const int st = make_plan(dims, num_kv_heads, &p);
  if (st != PA_OK) return st;
  memset(plan, 0, sizeof(*plan));
  plan->kernel = p.kernel;
  plan->partition_tokens = p.partition_tokens;
  plan->max_partitions = p.max_parts;
  plan->grid_workgroups = (int32_t)p.grid;
  plan->reduce_workgroups = (int32_t)p.reduce_grid;
  plan->schedule = p.schedule;
  plan->waves_per_item = p.waves_per_item;
  plan->workspace_bytes = p.ws_bytes;
  return PA_OK;
}

int pa_decode_ws(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                 const int32_t* seq_lens, int32_t num_kv_heads, float scale, void* out,
                 const pa_dims_t* dims, void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, dims, workspace,
             workspace_bytes, static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr);
}

int pa_decode_ws_timed(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens, int32_t num_kv_heads,
                       float scale, void* out, const pa_dims_t* dims, void* workspace,
                       size_t workspace_bytes, void* stream, void* ev_start, void* ev_mid,
                       void* ev_end) {
  return run(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, dims, workspace,
             workspace_bytes, static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev_start),
             static_cast<hipEvent_t>(ev_mid), static_cast<hipEvent_t>(ev_end));
}

int pa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
              const int32_t* seq_lens, int32_t num_kv_heads, float scale, void* out,
              const pa_dims_t* dims, void* stream) {
  Plan p;
  const int st = validate(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, dims, &p);
  if (st != PA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (p.ws_bytes > 0 && hipMallocAsync(&ws, p.ws_bytes, s) != hipSuccess) return PA_ERR_HIP;
  const int rc = run(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, dims, ws,
                     p.ws_bytes, s, nullptr, nullptr, nullptr);
  if (ws != nullptr && hipFreeAsync(ws, s) != hipSuccess && rc == PA_OK) return PA_ERR_HIP;
  return rc;
}

int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, int32_t num_kv_heads, float scale, void* out,
                      const pa_dims_t* dims, void* stream) {
  Plan p;
  const int st = validate(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, dims, &p);
  if (st != PA_OK) return st;
  if (p.ws_bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;   // before any HIP call
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int sst = scratch_for(s, &ws);
  if (sst != PA_OK) return sst;
  return run(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, dims, ws,
             (size_t)PA_NOALLOC_SCRATCH_BYTES, s, nullptr, nullptr, nullptr);
}

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid sizes (non-positive, num_heads % num_kv_heads, bounds, scale)";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: unsupported head_dim / block_size / group / dtype / kernel";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: q, caches and out need 16-byte alignment, tables and seq_lens 4";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing, too small or not 256-byte aligned";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown pa_decode status";
  }
}

int pa_version(void) { return (kVersionMajor << 16) | kVersionMinor; }

}  // extern "C"
