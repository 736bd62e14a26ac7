/*
 * pa_cache.h - writes into the paged KV cache on MI355X (gfx950): the append
 * that precedes every decode step and the copy-on-write block copy.
 *
 * Append ("Optimização da inferência" page, "Caches de KV": when token N is
 * generated only its key and value are computed and added to the cache;
 * vLLM e PagedAttention page: the block-table layout, and the fp8_e5m2 KV
 * option):
 *   for every new token i with sequence s = token_seq[i] and logical position
 *   p = token_pos[i] >= 0, block b = block_tables[s][p / block_size] and slot
 *   t = p % block_size:
 *       k_cache[b][g][d][t] = encode(k_new[i][g][d] / k_scale)
 *       v_cache[b][g][d][t] = encode(v_new[i][g][d] / v_scale)
 *   for every KV head g and d < head_dim. encode() is the identity for an
 *   fp32 cache fed fp32, and rounds to nearest even otherwise: bf16; OCP
 *   E5M2, where values beyond the largest finite code go to infinity; OCP
 *   E4M3 (no infinities), where values that round beyond 448 become NaN.
 *   For an fp8 cache the division is one correctly rounded fp32 division;
 *   for other caches the scales must be 1.
 *   INT4 cache (the inference page's exercise names INT4 KV; the format is
 *   the one of pa_decode.h): the code is the nearest integer to
 *   value / (k_scale * k_block_scales[b][g]) (the product rounded to fp32
 *   first, one fp32 division), ties to even, held to -8..7, NaN -> 0, stored
 *   as a two's-complement nibble (two tokens per byte, the even token in the
 *   low nibble). The same per-block scales may divide an fp8 cache's values.
 *   A negative token_pos marks a padding entry that writes nothing.
 *
 * Copy on write ("Optimização da inferência" page, "PagedAttention": pages
 * of a shared prefix are stored once; a request that diverges gets its own):
 *   for every pair i, physical block dst_blocks[i] of both caches (all KV
 *   heads, all slots) becomes a copy of block src_blocks[i], and so do its
 *   per-block scales when dims carries them.
 *
 * Layouts are those of pa_decode.h: caches [num_blocks][num_kv_heads]
 * [head_dim][block_size]; k_new / v_new [num_tokens][num_kv_heads][head_dim]
 * in in_dtype (F32 or BF16), contiguous, 16-byte aligned; token_seq,
 * token_pos, src_blocks, dst_blocks int32 device arrays.
 *
 * Ownership and errors as in pa_decode.h: caller-owned device memory, work
 * enqueued on `stream` (hipStream_t as void*) without synchronising, host-side
 * validation before any HIP call, a pa_status_t result.
 *
 * Caller's obligations on the buffers (sizes only cross this interface): the
 * caches hold num_blocks * num_kv_heads * head_dim * block_size elements of
 * kv_dtype (int4: two tokens per byte); k_new and v_new hold num_tokens rows of
 * [num_kv_heads][head_dim] with the caches' num_kv_heads and head_dim;
 * token_seq and token_pos hold num_tokens entries; block_tables num_seqs rows
 * of max_blocks_per_seq; src_blocks and dst_blocks num_pairs entries each. The
 * Python binding checks these against the tensors' shapes and raises
 * PA_ERR_SHAPE before calling the library.
 *
 * Device-side preconditions (not checked; violations are clamped or skipped
 * so every access stays in bounds, and the result is then unspecified):
 *   append: 0 <= token_seq[i] < num_seqs; token_pos[i] < max_blocks_per_seq *
 *           block_size; the table entries used are valid block ids; no two
 *           tokens write the same (block, slot).
 *   copy:   ids in [0, num_blocks); destinations distinct, and no block both
 *           a source and a destination.
 */
#ifndef PA_CACHE_H
#define PA_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dims: num_seqs, head_dim, num_blocks, block_size, max_blocks_per_seq,
 * kv_dtype (cache element type), k_scale, v_scale, k_block_scales,
 * v_block_scales are read; the rest ignored. Supported (in_dtype -> kv_dtype):
 * F32->F32, F32->BF16, BF16->BF16, F32 or BF16 -> FP8_E5M2, FP8_E4M3 or INT4
 * (INT4 requires both block-scale arrays; fp8 takes both or neither; the
 * scales themselves are read, never written); head_dim 64 or 128; block_size
 * 16. A run of list entries that covers a whole block in order is written
 * row by row with wide stores; the result is the same as token by token. */
int pa_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* block_tables, const int32_t* token_seq,
                    const int32_t* token_pos, int32_t num_tokens, int32_t num_kv_heads,
                    int32_t in_dtype, const pa_dims_t* dims, void* stream);

/* dims: head_dim, num_blocks, block_size, kv_dtype, k_block_scales,
 * v_block_scales are read (the scale arrays, when given, are copied with
 * their blocks). num_pairs may be 0. */
int pa_cache_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t num_pairs, int32_t num_kv_heads,
                         const pa_dims_t* dims, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_CACHE_H */
