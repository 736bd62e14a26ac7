// Writes into the paged KV cache (gfx950): the per-step append of new
// tokens' K/V through the block table, with encoding to the cache type, and
// the copy-on-write block copy. Both are small memory-bound scatters/copies;
// the append's stores follow the cache layout, whose tokens are the fastest
// axis, so one token touches one element in each head_dim row.

#include <math.h>

#include "pa_cache.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// float -> OCP E5M2, round to nearest even, overflow to infinity, NaN kept.
__device__ __forceinline__ uint8_t f32_to_e5m2(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return static_cast<uint8_t>(sign | 0x7Fu);      // NaN
  if (a >= 0x47700000u) return static_cast<uint8_t>(sign | 0x7Cu);     // |x| >= 61440 rounds past 57344
  if (a >= 0x38800000u) {                                               // |x| >= 2^-14: normal code
    const uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);                 // keep 2 mantissa bits, ties to even
    return static_cast<uint8_t>(sign | ((r >> 21) - (112u << 2)));      // rebias 127 -> 15
  }
  // subnormal step 2^-16; the scaling is exact and rint rounds ties to even
  const float q = rintf(__uint_as_float(a) * 65536.0f);
  return static_cast<uint8_t>(sign | static_cast<uint32_t>(q));
}

// float -> OCP E4M3, round to nearest even; no infinities: magnitudes above
// 464 (which round past 448), infinities and NaN give the NaN code.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x43E80000u) return static_cast<uint8_t>(sign | 0x7Fu);      // > 464, inf, NaN
  if (a >= 0x3C800000u) {                                               // |x| >= 2^-6: normal code
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);                 // keep 3 mantissa bits, ties to even
    return static_cast<uint8_t>(sign | ((r >> 20) - (120u << 3)));      // rebias 127 -> 7
  }
  const float q = rintf(__uint_as_float(a) * 512.0f);                   // subnormal step 2^-9
  return static_cast<uint8_t>(sign | static_cast<uint32_t>(q));
}

// float -> int4 code: nearest integer, ties to even, held to -8..7; NaN gives 0.
__device__ __forceinline__ uint32_t f32_to_int4_nibble(float y) {
  if (y != y) return 0u;
  const float r = fminf(fmaxf(rintf(y), -8.0f), 7.0f);
  return static_cast<uint32_t>(static_cast<int>(r)) & 0xFu;
}

template <int IN> __device__ __forceinline__ float load_in(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_in<kF32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load_in<kBF16>(const void* p, int64_t i) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int KV> __device__ __forceinline__ void store_kv(void* cache, int64_t i, float x, float scale);
template <> __device__ __forceinline__ void store_kv<kF32>(void* cache, int64_t i, float x, float) {
  static_cast<float*>(cache)[i] = x;
}
template <> __device__ __forceinline__ void store_kv<kBF16>(void* cache, int64_t i, float x, float) {
  static_cast<uint16_t*>(cache)[i] = f32_to_bf16_bits(x);
}
template <> __device__ __forceinline__ void store_kv<kE5M2>(void* cache, int64_t i, float x, float scale) {
  static_cast<uint8_t*>(cache)[i] = f32_to_e5m2(x / scale);
}
template <> __device__ __forceinline__ void store_kv<kE4M3>(void* cache, int64_t i, float x, float scale) {
  static_cast<uint8_t*>(cache)[i] = f32_to_e4m3(x / scale);
}
// int4: element i is nibble i & 1 of byte i / 2. Another token of the same call
// may own the other nibble (or a neighbouring byte of the same word), so the
// nibble is cleared and set with two atomics on its 32-bit word, which leave
// every other nibble alone.
template <> __device__ __forceinline__ void store_kv<kI4>(void* cache, int64_t i, float x, float scale) {
  const int64_t byte = i >> 1;
  unsigned int* word = reinterpret_cast<unsigned int*>(static_cast<uint8_t*>(cache) + (byte & ~int64_t(3)));
  const uint32_t shift = uint32_t(byte & 3) * 8u + uint32_t(i & 1) * 4u;
  atomicAnd(word, ~(0xFu << shift));
  atomicOr(word, f32_to_int4_nibble(x / scale) << shift);
}

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* tables;
  const int32_t* token_seq;
  const int32_t* token_pos;
  int32_t num_tokens, num_kv_heads, head_dim, num_seqs, max_blocks, num_blocks;
  float k_scale, v_scale;
  const float* k_bscale;   // per-(block, KV head) scales, or null
  const float* v_bscale;
};

// Code bits of one value for a whole-row store.
template <int KV> __device__ __forceinline__ uint32_t encode(float x, float scale);
template <> __device__ __forceinline__ uint32_t encode<kF32>(float x, float) { return __float_as_uint(x); }
template <> __device__ __forceinline__ uint32_t encode<kBF16>(float x, float) { return f32_to_bf16_bits(x); }
template <> __device__ __forceinline__ uint32_t encode<kE5M2>(float x, float scale) { return f32_to_e5m2(x / scale); }
template <> __device__ __forceinline__ uint32_t encode<kE4M3>(float x, float scale) { return f32_to_e4m3(x / scale); }
template <> __device__ __forceinline__ uint32_t encode<kI4>(float x, float scale) {
  return f32_to_int4_nibble(x / scale);
}

// One head_dim row of a block tile (16 tokens) from 16 encoded values, written
// with 128-bit stores (64-bit for int4). `row` is the row's first element.
template <int KV> __device__ __forceinline__ void store_row(void* cache, int64_t row, const uint32_t (&c)[16]) {
  constexpr int kBits = KV == kF32 ? 32 : KV == kBF16 ? 16 : KV == kI4 ? 4 : 8;
  uint32_t w[16 * kBits / 32];
#pragma unroll
  for (int k = 0; k < 16 * kBits / 32; ++k) {
    w[k] = 0;
#pragma unroll
    for (int e = 0; e < 32 / kBits; ++e) w[k] |= c[k * (32 / kBits) + e] << (e * kBits);
  }
  char* dst = static_cast<char*>(cache) + row * kBits / 8;
  if constexpr (kBits == 4) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int k = 0; k < 16 * kBits / 32; k += 4)
      *reinterpret_cast<uint4*>(dst + 4 * k) = make_uint4(w[k], w[k + 1], w[k + 2], w[k + 3]);
  }
}

// One wavefront per (list entry, KV head). If the entry's block is written
// whole by this call (the 16 entries from the one at the block's first
// position are that block's positions, in order, in the same sequence: a bulk
// append), the wavefront of that first entry writes the block, lane d rows d
// and d + 64, 16 tokens each, with wide stores, and the other 15 return.
// Otherwise lane d writes element (d, slot) of rows d and d + 64 (int4: one
// nibble, by atomics on its word).
//
// The (sequence, position) pairs of the entry and of the 15 on either side,
// which the check needs, arrive in one round of loads, one entry per lane:
// most wavefronts of a bulk append only find that another writes their
// block, and their time is that round.
template <int IN, int KV>
__global__ __launch_bounds__(64) void append_kernel(const AppendArgs a) {
  constexpr int kHalo = kBlockSize - 1;
  const int i = blockIdx.x;
  const int g = blockIdx.y;
  const int lane = threadIdx.x;
  const int we = i - kHalo + lane;                  // entry of this lane's window slot
  const bool in_win = lane < 2 * kHalo + 1 && we >= 0 && we < a.num_tokens;
  const int wseq = in_win ? a.token_seq[we] : -1;
  const int wpos = in_win ? a.token_pos[we] : -1;
  const int s = __builtin_amdgcn_readlane(wseq, kHalo);
  const int pos = __builtin_amdgcn_readlane(wpos, kHalo);
  const int max_pos = a.max_blocks * kBlockSize;
  if (pos < 0 || s < 0 || s >= a.num_seqs || pos >= max_pos) return;
  const int slot = pos % kBlockSize;
  const int first = i - slot;                       // list index of the block's first position, if bulk
  bool whole = false;
  if (first >= 0 && first + kBlockSize <= a.num_tokens && pos - slot + kBlockSize <= max_pos) {
    const int k = lane - (kHalo - slot);            // this lane's entry is first + k
    const bool ok = k < 0 || k >= kBlockSize || (wseq == s && wpos == pos - slot + k);
    whole = __builtin_amdgcn_ballot_w64(!ok) == 0;
  }
  if (whole && slot != 0) return;                   // written by the block's first entry
  // Runs (not int4): entries that continue the previous entry's sequence at
  // the next position of the same block are written by the wavefront of the
  // run's first entry, which writes the run's tokens row after row; so each
  // row's bytes of the run are stored back to back by one wavefront and reach
  // the L2 together (otherwise the partial last block of every sequence in a
  // bulk append is written two bytes per row by separate wavefronts, and L2
  // writes some of its sectors back more than once). Other runs in the same
  // block hold other slots: their bytes are disjoint.
  int run = 1;                                      // entries of this entry's run from it on
  if constexpr (KV != kI4) {
    if (!whole) {
      const bool pred = slot > 0 && __builtin_amdgcn_readlane(wseq, kHalo - 1) == s &&
                        __builtin_amdgcn_readlane(wpos, kHalo - 1) == pos - 1;
      if (pred) return;                             // written by the run's first entry
      const int k = lane - kHalo;                   // this lane's entry is i + k
      const bool next = k >= 1 && k < kBlockSize - slot && wseq == s && wpos == pos + k;
      const uint64_t m = __builtin_amdgcn_ballot_w64(next) >> (kHalo + 1);   // bit j: entry i + 1 + j
      run = 1 + __builtin_ctzll(~m);                // consecutive successors inside the block
    }
  }
  int32_t id = a.tables[(int64_t)s * a.max_blocks + pos / kBlockSize];
  id = min(max(id, 0), a.num_blocks - 1);
  // code of value / scale, the scale being k_scale times the block's own
  // (rounded to float32 first) when the cache has per-block scales
  const float ks = a.k_bscale ? a.k_scale * a.k_bscale[(int64_t)id * a.num_kv_heads + g] : a.k_scale;
  const float vs = a.v_bscale ? a.v_scale * a.v_bscale[(int64_t)id * a.num_kv_heads + g] : a.v_scale;
  const int64_t head_stride = (int64_t)a.num_kv_heads * a.head_dim;   // elements per list entry
  const int64_t src = (int64_t)i * head_stride + (int64_t)g * a.head_dim;
  const int64_t tile = ((int64_t)id * a.num_kv_heads + g) * a.head_dim * kBlockSize;   // in elements
  if (whole) {
    for (int d = lane; d < a.head_dim; d += 64) {
      uint32_t ck[kBlockSize], cv[kBlockSize];
#pragma unroll
      for (int t = 0; t < kBlockSize; ++t) {
        ck[t] = encode<KV>(load_in<IN>(a.k_new, src + t * head_stride + d), ks);
        cv[t] = encode<KV>(load_in<IN>(a.v_new, src + t * head_stride + d), vs);
      }
      store_row<KV>(a.k_cache, tile + (int64_t)d * kBlockSize, ck);
      store_row<KV>(a.v_cache, tile + (int64_t)d * kBlockSize, cv);
    }
    return;
  }
  if (run > 1) {
    // four tokens at a time (their loads in flight together), a row's stores back to back
    for (int d = lane; d < a.head_dim; d += 64) {
      for (int t0 = 0; t0 < run; t0 += 4) {
        float kx[4], vx[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int tt = min(t0 + t, run - 1);   // past the run: reload its last token, not stored
          kx[t] = load_in<IN>(a.k_new, src + tt * head_stride + d);
          vx[t] = load_in<IN>(a.v_new, src + tt * head_stride + d);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t0 + t < run) {
            store_kv<KV>(a.k_cache, tile + (int64_t)d * kBlockSize + slot + t0 + t, kx[t], ks);
            store_kv<KV>(a.v_cache, tile + (int64_t)d * kBlockSize + slot + t0 + t, vx[t], vs);
          }
        }
      }
    }
    return;
  }
  for (int d = lane; d < a.head_dim; d += 64) {
    store_kv<KV>(a.k_cache, tile + (int64_t)d * kBlockSize + slot, load_in<IN>(a.k_new, src + d), ks);
    store_kv<KV>(a.v_cache, tile + (int64_t)d * kBlockSize + slot, load_in<IN>(a.v_new, src + d), vs);
  }
}

struct CopyArgs {
  char* k_cache;
  char* v_cache;
  const int32_t* src;
  const int32_t* dst;
  int64_t block_bytes;   // one physical block, all KV heads
  int32_t num_blocks;
  int32_t num_kv_heads;
  float* k_bscale;       // per-(block, KV head) scales copied with their blocks, or null
  float* v_bscale;
};

constexpr int kCopyThreads = 256;
constexpr int kCopyChunk = kCopyThreads * 16;   // bytes per workgroup

// Grid (pair, chunk of the block, cache): 128-bit loads and stores.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const CopyArgs a) {
  const int i = blockIdx.x;
  const int64_t off = (int64_t)blockIdx.y * kCopyChunk + (int64_t)threadIdx.x * 16;
  if (off >= a.block_bytes) return;
  const int64_t sb = min(max(a.src[i], 0), a.num_blocks - 1);
  const int64_t db = min(max(a.dst[i], 0), a.num_blocks - 1);
  char* base = blockIdx.z == 0 ? a.k_cache : a.v_cache;
  const uint4 x = *reinterpret_cast<const uint4*>(base + sb * a.block_bytes + off);
  *reinterpret_cast<uint4*>(base + db * a.block_bytes + off) = x;
  if (a.k_bscale != nullptr && blockIdx.y == 0) {
    float* sc = blockIdx.z == 0 ? a.k_bscale : a.v_bscale;
    for (int g = threadIdx.x; g < a.num_kv_heads; g += kCopyThreads)
      sc[db * a.num_kv_heads + g] = sc[sb * a.num_kv_heads + g];
  }
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

int elem_bits(int dtype) { return dtype == kF32 ? 32 : dtype == kBF16 ? 16 : dtype == kI4 ? 4 : 8; }

int check_cache_dims(const pa_dims_t* d, int32_t hkv) {
  if (d == nullptr) return PA_ERR_NULL;
  if (d->head_dim <= 0 || d->num_blocks <= 0 || d->block_size <= 0 || hkv <= 0) return PA_ERR_SHAPE;
  if (d->block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (d->kv_dtype != kF32 && d->kv_dtype != kBF16 && d->kv_dtype != kE5M2 && d->kv_dtype != kE4M3 &&
      d->kv_dtype != kI4)
    return PA_ERR_UNSUPPORTED;
  if (hkv > 65535) return PA_ERR_UNSUPPORTED;
  // per-block scales: both or neither; required for int4, allowed for fp8
  if ((d->k_block_scales == nullptr) != (d->v_block_scales == nullptr)) return PA_ERR_NULL;
  if (d->kv_dtype == kI4 && d->k_block_scales == nullptr) return PA_ERR_NULL;
  if (d->k_block_scales != nullptr && (d->kv_dtype == kF32 || d->kv_dtype == kBF16)) return PA_ERR_UNSUPPORTED;
  if (!aligned(d->k_block_scales, 4) || !aligned(d->v_block_scales, 4)) return PA_ERR_ALIGN;
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" int pa_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const int32_t* block_tables, const int32_t* token_seq,
                               const int32_t* token_pos, int32_t num_tokens, int32_t num_kv_heads,
                               int32_t in_dtype, const pa_dims_t* dims, void* stream) {
  int st = check_cache_dims(dims, num_kv_heads);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || dims->num_seqs <= 0 || dims->max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  const int kv = dims->kv_dtype;
  const bool fp8 = kv == kE5M2 || kv == kE4M3 || kv == kI4;   // coded caches: value / scale is encoded
  const bool combo = (in_dtype == kF32 && (kv == kF32 || kv == kBF16 || fp8)) || (in_dtype == kBF16 && (kv == kBF16 || fp8));
  if (!combo) return PA_ERR_UNSUPPORTED;
  if (!isfinite(dims->k_scale) || !isfinite(dims->v_scale) || dims->k_scale == 0.f || dims->v_scale == 0.f)
    return PA_ERR_SHAPE;
  if (!fp8 && (dims->k_scale != 1.f || dims->v_scale != 1.f)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !token_seq || !token_pos) return PA_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(token_seq, 4) || !aligned(token_pos, 4))
    return PA_ERR_ALIGN;
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.token_seq = token_seq;
  a.token_pos = token_pos;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = dims->head_dim;
  a.num_seqs = dims->num_seqs;
  a.max_blocks = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  a.k_scale = dims->k_scale;
  a.v_scale = dims->v_scale;
  a.k_bscale = dims->k_block_scales;
  a.v_bscale = dims->v_block_scales;
  const dim3 grid(num_tokens, num_kv_heads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (in_dtype == kF32 && kv == kF32) append_kernel<kF32, kF32><<<grid, 64, 0, s>>>(a);
  else if (in_dtype == kF32 && kv == kBF16) append_kernel<kF32, kBF16><<<grid, 64, 0, s>>>(a);
  else if (in_dtype == kF32 && kv == kE5M2) append_kernel<kF32, kE5M2><<<grid, 64, 0, s>>>(a);
  else if (in_dtype == kBF16 && kv == kBF16) append_kernel<kBF16, kBF16><<<grid, 64, 0, s>>>(a);
  else if (in_dtype == kF32 && kv == kE4M3) append_kernel<kF32, kE4M3><<<grid, 64, 0, s>>>(a);
  else if (in_dtype == kBF16 && kv == kE5M2) append_kernel<kBF16, kE5M2><<<grid, 64, 0, s>>>(a);
  else if (in_dtype == kBF16 && kv == kE4M3) append_kernel<kBF16, kE4M3><<<grid, 64, 0, s>>>(a);
  else if (in_dtype == kF32 && kv == kI4) append_kernel<kF32, kI4><<<grid, 64, 0, s>>>(a);
  else append_kernel<kBF16, kI4><<<grid, 64, 0, s>>>(a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" int pa_cache_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                                    const int32_t* dst_blocks, int32_t num_pairs, int32_t num_kv_heads,
                                    const pa_dims_t* dims, void* stream) {
  int st = check_cache_dims(dims, num_kv_heads);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks) return PA_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(src_blocks, 4) || !aligned(dst_blocks, 4))
    return PA_ERR_ALIGN;
  CopyArgs a;
  a.k_cache = static_cast<char*>(k_cache);
  a.v_cache = static_cast<char*>(v_cache);
  a.src = src_blocks;
  a.dst = dst_blocks;
  a.block_bytes = (int64_t)num_kv_heads * dims->head_dim * dims->block_size * elem_bits(dims->kv_dtype) / 8;
  a.num_blocks = dims->num_blocks;
  a.num_kv_heads = num_kv_heads;
  // the scale arrays travel with their blocks; the copy writes them
  a.k_bscale = const_cast<float*>(dims->k_block_scales);
  a.v_bscale = const_cast<float*>(dims->v_block_scales);
  const dim3 grid(num_pairs, (unsigned)((a.block_bytes + kCopyChunk - 1) / kCopyChunk), 2);
  copy_blocks_kernel<<<grid, kCopyThreads, 0, static_cast<hipStream_t>(stream)>>>(a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
