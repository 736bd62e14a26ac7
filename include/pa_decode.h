/*
 * pa_decode.h - PagedAttention decode on AMD Instinct MI355X (gfx950).
 *
 * The operation (vLLM e PagedAttention page, PagedAttention kernel pseudocode;
 * "Optimização da inferência" page, step 2, attention with the KV cache):
 *
 *   for every sequence s and query head h, with L = seq_lens[s] and
 *   KV head g = h / (num_heads / num_kv_heads):
 *       token t < L of sequence s is stored in physical block
 *       block_tables[s][t / block_size], slot t % block_size;
 *       out[s][h][:] = sum_t softmax_t(scale * q[s][h] . K_t) * V_t
 *   and out[s][h][:] = 0 when L == 0.
 *
 * The kernels accumulate the softmax online (running max, running sum,
 * rescaled output) over whole physical blocks, split long sequences into
 * context partitions and merge the partitions in a second kernel.
 *
 * Layouts (all row-major, contiguous, every pointer 16-byte aligned):
 *   q, out        [num_seqs][num_heads][head_dim]                  element type q_dtype
 *   k_cache       [num_blocks][num_kv_heads][head_dim][block_size] element type kv_dtype
 *   v_cache       same as k_cache
 *   block_tables  [num_seqs][max_blocks_per_seq]                   int32 physical block ids
 *   seq_lens      [num_seqs]                                       int32
 * (the cache layout is the one in the kernel pseudocode; its head axis counts
 *  KV heads, as the KV-cache size formula on the inference page does.)
 *
 * Ownership: every data pointer is caller-owned device memory. The library
 * never frees it, keeps no reference after the call returns, and never
 * synchronises the device or the stream. Work is enqueued on `stream` (a
 * hipStream_t passed as void*, NULL = the default stream); inputs must stay
 * alive, and `out` untouched, until the stream reaches that point. q, the
 * caches, the tables and seq_lens are only read; out is only written.
 *
 * Errors: every call returns a pa_status_t. Argument validation happens on
 * the host before any HIP call, so a rejected call enqueues nothing. There is
 * no global error state; pa_status_str() names a status.
 *
 * Caller's obligations on the buffers (this interface receives sizes, not
 * allocations, so it cannot check them; a mismatch is an out-of-bounds access):
 * each cache holds num_blocks * num_kv_heads * head_dim * block_size elements
 * in the layout above, i.e. its KV-head axis has exactly num_kv_heads entries
 * and its head_dim axis is q's; q and out hold num_seqs * q_len * num_heads *
 * head_dim elements; block_tables num_seqs rows of max_blocks_per_seq; seq_lens
 * num_seqs entries; per-block scale arrays num_blocks * num_kv_heads floats.
 * The Python binding compares these with the tensors' shapes (and the element
 * size with kv_dtype) and raises PA_ERR_SHAPE before calling the library.
 *
 * Device-side preconditions (not checked, the data lives on the device):
 *   0 <= seq_lens[s] <= min(max_seq_len, max_blocks_per_seq * block_size)
 *   0 <= block_tables[s][j] < num_blocks for j < ceil(seq_lens[s] / block_size)
 * Table entries past ceil(seq_lens[s] / block_size), and cache slots past
 * seq_lens[s] in the last block, are never read. Several sequences may map
 * to the same physical block (shared prefixes).
 *
 * Scales: scale and k_scale must be positive and finite, and so must their
 * product with log2(e) (the kernels work in the log2 domain); v_scale finite.
 * Otherwise the call returns PA_ERR_SHAPE.
 *
 * Numeric range. Every kernel accumulates in float32 and needs the scores
 * scale * k_scale * (block scale) * q . K to be finite in float32. The
 * matrix-core kernel's fp8 and int4 paths multiply binary16 operands; they
 * take any finite bf16 q and any per-block scale in [2^-100, 2^100] without
 * loss of range:
 *   - each (query position, head) row of q is multiplied by the power of two
 *     that puts its largest magnitude in [2^14, 2^15) before rounding to
 *     binary16 (exact for every element down to 2^-28 of that maximum), and
 *     its scores are multiplied back in float32; this requires
 *     |scale * k_scale * k_block_scale| * max|q| < 2^100;
 *   - a per-block V scale is split into a mantissa in [1, 2), which multiplies
 *     the softmax weights fed to the matrix cores (kept in [0, 2)), and a power
 *     of two, added to the score in the log2 domain, so the running maximum
 *     follows weight x scale and no fed weight overflows or loses precision.
 * Softmax weights in the P.V product. Decode (q_len = 1) with a bf16 cache
 * feeds each weight as a rounded bf16 value plus its rounding residual (about
 * 16 significant bits). Calls with more than 16 (query position, head) pairs
 * per KV head (several query positions per sequence) and decode with an fp8
 * or int4 cache feed the rounded value alone: 8 significant bits (bf16 cache)
 * or 11 (binary16: fp8, int4), which moves an output by at most 2^-9 (2^-12)
 * of sum_i p_i |v_i|, well inside the stated bars (2e-2 for bf16 I/O, 5e-2
 * for fp8 KV).
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                              */
  PA_ERR_SHAPE = 2,       /* non-positive size or scale, num_heads % num_kv_heads,   */
  PA_ERR_UNSUPPORTED = 3, /* head_dim / block_size / group / dtype combination       */
  PA_ERR_ALIGN = 4,       /* a data pointer is not 16-byte aligned                   */
  PA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than pa_decode_workspace_bytes */
  PA_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed              */
} pa_status_t;

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_BF16 = 1,      /* bfloat16; outputs rounded to nearest even              */
  PA_DTYPE_FP8_E5M2 = 2,  /* OCP E5M2 (bias 15, IEEE-style inf/NaN); KV cache only  */
  PA_DTYPE_FP8_E4M3 = 3,  /* OCP E4M3 (bias 7, no inf, S.1111.111 NaN); KV cache only */
  PA_DTYPE_INT4 = 4       /* two's-complement codes -8..7, two tokens per byte (the
                             even token in the low nibble), so a block row of 16
                             tokens is 8 bytes; values are code * k_scale (v_scale) *
                             the block's scale (k_block_scales / v_block_scales,
                             required). KV cache only, matrix-core kernel. The
                             inference page's exercise names INT4 KV quantisation and
                             its fourfold capacity over FP16; format and scale
                             granularity are this library's reading.             */
} pa_dtype_t;

typedef enum pa_schedule {
  PA_SCHEDULE_AUTO = 0,   /* queue when the dense grid far exceeds the resident waves */
  PA_SCHEDULE_GRID = 1,   /* one workgroup per (KV head, sequence, partition)          */
  PA_SCHEDULE_QUEUE = 2   /* a plan kernel lists the non-empty items, longest first,
                             and workgroup i takes item i (matrix-core kernel,
                             partitions of at most 8192 tokens)                     */
} pa_schedule_t;

typedef enum pa_kernel {
  PA_KERNEL_AUTO = 0,     /* matrix-core kernel where supported, else vector kernel  */
  PA_KERNEL_VALU = 1,     /* vector-ALU kernel (every supported shape)               */
  PA_KERNEL_MFMA = 2      /* matrix-core kernel: head_dim 128, block 16, any group,
                             q_len <= 4096, q bf16 with KV bf16, fp8 or int4        */
} pa_kernel_t;

/* Sizes and types of one call. Supported: block_size 16; head_dim 64 or 128;
 * group = num_heads / num_kv_heads in {1, 2, 4, 8, 16} (any group for the
 * matrix-core kernel); (q_dtype, kv_dtype) in {(F32, F32), (BF16, BF16),
 * (BF16, FP8_E5M2), (BF16, FP8_E4M3), (BF16, INT4)} (INT4 and per-block scales:
 * matrix-core kernel, head_dim 128).
 * Non-finite K/V values in attended slots give non-finite outputs (the
 * matrix-core kernel may return NaN where exact arithmetic gives +-inf). */
typedef struct pa_dims {
  int32_t num_seqs;
  int32_t num_heads;           /* query heads                                         */
  int32_t head_dim;
  int32_t num_blocks;          /* physical blocks in each cache                        */
  int32_t block_size;          /* tokens per block                                     */
  int32_t max_blocks_per_seq;  /* block_tables row length                              */
  int32_t q_dtype;             /* pa_dtype_t of q and out                              */
  int32_t kv_dtype;            /* pa_dtype_t of k_cache and v_cache                    */
  float k_scale;               /* per-tensor dequantisation scales (1.0f unless fp8)   */
  float v_scale;
  int32_t max_seq_len;         /* host upper bound on seq_lens, sizes the split grid;
                                  0 means max_blocks_per_seq * block_size             */
  int32_t partition_tokens;    /* context-partition length; 0 = chosen by the library,
                                  else a positive multiple of 64                      */
  int32_t kernel;              /* pa_kernel_t                                          */
  int32_t q_len;               /* query positions per sequence; 0 or 1 = decode. With
                                  q_len > 1, q and out are [num_seqs][q_len][num_heads]
                                  [head_dim], seq_lens count the q_len new tokens, and
                                  query i attends tokens t < seq_lens[s] - q_len + 1 + i
                                  (the causal mask of the inference page's attention
                                  with several query rows; a query with no token gets
                                  a zero row). Matrix-core kernel only, q_len <= 4096:
                                  a KV head's group * q_len (position, head) pairs
                                  are taken in blocks of up to 64 per work item. With
                                  more, the waves of a work item take 32 pairs each
                                  and read every K/V tile once, through LDS (see
                                  waves_per_item).                                   */
  int32_t schedule;            /* pa_schedule_t                                        */
  int32_t waves_per_item;      /* matrix-core kernel: waves that share one (sequence,
                                  KV head, partition) item; 0 = chosen by the library.
                                  group * q_len <= 64: the waves split the item's
                                  tiles and merge their states in LDS: 1, 2, 3 or 4
                                  (3 and 4 only with group * q_len <= 16). group *
                                  q_len > 64:
                                  2, 4 or 8 waves take 32 (query position, head)
                                  pairs each and share every K/V tile through LDS
                                  (default: 2 for up to 64 pairs, else 4; 8 with a
                                  bf16 cache past 4096 tokens and more than 128
                                  pairs); 1 gives
                                  one block of 64 pairs per item, each block reading
                                  the tiles itself.                                  */
  const float* k_block_scales; /* device, [num_blocks][num_kv_heads] float32: the K
                                  values of physical block b, KV head g are multiplied
                                  by k_block_scales[b * num_kv_heads + g]. Required for
                                  INT4, optional (NULL) for FP8, NULL otherwise; only
                                  entries of blocks the tables reference are read
                                  (matrix-core kernel). 4-byte aligned.              */
  const float* v_block_scales; /* the same for V                                      */
} pa_dims_t;

/* Decode with a workspace the library takes from the stream-ordered allocator
 * (hipMallocAsync / hipFreeAsync on `stream`) when the plan needs one. */
int pa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens,
              int32_t num_kv_heads, float scale, void* out,
              const pa_dims_t* dims, void* stream);

/* Bytes of device workspace pa_decode_ws needs for these sizes (0 if none).
 * Returns 0 and sets *status (if non-NULL) on invalid arguments. */
size_t pa_decode_workspace_bytes(const pa_dims_t* dims, int32_t num_kv_heads, int* status);

/* Decode with a caller-owned device workspace of at least
 * pa_decode_workspace_bytes() bytes, 256-byte aligned. The workspace holds the
 * per-partition softmax states between the two kernels; it may be reused by
 * the next call on the same stream. */
int pa_decode_ws(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens,
                 int32_t num_kv_heads, float scale, void* out,
                 const pa_dims_t* dims, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): pa_decode
 * with the workspace taken from a fixed device array inside the library, one
 * per GPU, of PA_NOALLOC_SCRATCH_BYTES, held until the process ends. It calls
 * no allocator. A call whose plan needs more (pa_decode_workspace_bytes)
 * returns PA_ERR_WORKSPACE before any HIP call. 128 MiB holds the partition
 * states of 256 sequences x 8 KV heads x 8 query heads at 32K tokens (65 MiB),
 * or 16 query positions of 16 such sequences (65 MiB). Every call on
 * one GPU uses that GPU's same array: calls that may overlap on a GPU (other
 * streams, other host threads) race and must be ordered by the caller; calls
 * on one stream are ordered by it. Results are those of pa_decode_ws with the
 * same arguments (same kernels, same plan). The array's device address is
 * looked up on the first call on each GPU (the stream's device). */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)
int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens,
                      int32_t num_kv_heads, float scale, void* out,
                      const pa_dims_t* dims, void* stream);

/* pa_decode_ws that also records three caller-created HIP events (hipEvent_t
 * as void*) on `stream`: ev_start and ev_mid at the start and end of the
 * partition kernel's execution (for the matrix-core kernel they are attached
 * to its dispatch, so they add no separate stream operations), ev_end after
 * the reduce kernel. Any event may be NULL. With the list schedule the plan
 * kernel runs before ev_start. */
int pa_decode_ws_timed(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens,
                       int32_t num_kv_heads, float scale, void* out,
                       const pa_dims_t* dims, void* workspace, size_t workspace_bytes,
                       void* stream, void* ev_start, void* ev_mid, void* ev_end);

/* The launch plan the library would use for these sizes (host only). */
typedef struct pa_plan {
  int32_t kernel;              /* pa_kernel_t actually used (never AUTO)              */
  int32_t partition_tokens;    /* tokens per context partition                         */
  int32_t max_partitions;      /* partitions of the longest allowed sequence           */
  int32_t grid_workgroups;     /* workgroups of the partition kernel                   */
  int32_t reduce_workgroups;   /* workgroups of the reduce kernel (0 = not launched)   */
  int32_t schedule;            /* pa_schedule_t actually used (never AUTO)             */
  int32_t waves_per_item;      /* waves per work item actually used                    */
  int32_t pad;
  size_t workspace_bytes;
} pa_plan_t;

int pa_decode_plan(const pa_dims_t* dims, int32_t num_kv_heads, pa_plan_t* plan);

/* Static description of a status code. */
const char* pa_status_str(int status);

/* Library version, (major << 16) | minor. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
