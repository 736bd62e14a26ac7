// Vector-ALU PagedAttention decode partition kernel (gfx950, wave64).
//
// One workgroup of one wavefront handles one (sequence, KV head, context
// partition) and all G query heads that share the KV head, so every K/V tile
// is read once per KV head (grouped-query sharing; the KV-cache size on the
// "Optimização da inferência" page counts KV heads, 64 query heads over 8).
// It walks the partition's logical blocks through the block table and keeps
// the online-softmax state (running max m, running sum l, rescaled o) of the
// PagedAttention kernel pseudocode on the vLLM page in registers.
//
// For small groups (G x head_dim / 4 <= 32) blocks are fetched ahead: the
// partition's physical block ids are read one per lane (64 at a time) and
// handed out with readlane, and the K and V tiles of block j + kDepth - 1 are
// issued, into a ring of raw registers, before block j is computed. A short
// sequence then costs about one memory round trip per kDepth blocks instead
// of three per block (id, then K, then V).
//
// Per 16-token block (tile [head_dim][16], tokens fastest):
//   QK: lane = (token t = lane % 16, row group c = lane / 16); the lane reads
//       rows d = 4i + c (one 128-byte line per wave instruction), multiplies
//       by q from LDS, and the four row groups are summed with two xor
//       shuffles. Every lane then holds the full score of its token.
//   softmax: max and sum over the 16 tokens with xor shuffles; scores are in
//       the log2 domain (scale * log2 e folded into one factor), so exp2.
//   PV: lane = row d (head_dim / 64 rows per lane), 16-token rows read with
//       128-bit loads, p broadcast from LDS.
// Token slots past the sequence end are selected out of the max, the sum and
// P.V (their bytes may be anything, NaN included).
//
// This kernel covers every supported shape and dtype; the matrix-core kernel
// replaces it for the grouped bf16 / fp8 shapes.


#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// A V row of 16 tokens is sizeof(element) x 16 bytes: that many 16-byte
// pieces, loaded raw and widened at use.
template <int KDT> struct Row16 {
  static constexpr int kPieces = (int)sizeof(typename Storage<KDT>::type);
  typedef uint4 raw_t[kPieces];
  static __device__ __forceinline__ void load(const void* row, raw_t& x) {
    const uint4* p = static_cast<const uint4*>(row);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) x[i] = p[i];
  }
  static __device__ __forceinline__ void widen(const raw_t& x, float (&v)[16]);
};

template <> __device__ __forceinline__ void Row16<kF32>::widen(const raw_t& x, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i + 0] = __uint_as_float(x[i].x); v[4 * i + 1] = __uint_as_float(x[i].y);
    v[4 * i + 2] = __uint_as_float(x[i].z); v[4 * i + 3] = __uint_as_float(x[i].w);
  }
}

template <> __device__ __forceinline__ void Row16<kBF16>::widen(const raw_t& x, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

template <> __device__ __forceinline__ void Row16<kE5M2>::widen(const raw_t& x, float (&v)[16]) {
  const uint32_t w[4] = {x[0].x, x[0].y, x[0].z, x[0].w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int b = 0; b < 4; ++b) v[4 * j + b] = e5m2_to_f32(w[j] >> (8 * b));
  }
}

template <> __device__ __forceinline__ void Row16<kE4M3>::widen(const raw_t& x, float (&v)[16]) {
  const uint32_t w[4] = {x[0].x, x[0].y, x[0].z, x[0].w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);   // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);    // bytes 2, 3
    v[4 * j + 0] = lo[0]; v[4 * j + 1] = lo[1]; v[4 * j + 2] = hi[0]; v[4 * j + 3] = hi[1];
  }
}

template <int QDT, int KDT, int D, int G>
__global__ __launch_bounds__(64) void valu_partition_kernel(const Args a) {
  using KT = typename Storage<KDT>::type;
  using QT = typename Storage<QDT>::type;
  constexpr int BS = kBlockSize;
  constexpr int DPL = D / 64;

  const Item item = work_item(a);
  const int part = item.part;
  const int kvh = item.kvh;
  const int s = item.s;
  const int lane = threadIdx.x;
  const int L = clamp_len(a, s);
  const int P = a.partition_tokens;
  const int nparts = L > 0 ? (L + P - 1) / P : 1;
  if (part >= nparts) return;
  const int tok0 = part * P;
  const int tok1 = min(L, tok0 + P);

  __shared__ float q_s[D][G];
  __shared__ float p_s[G][BS];

  const QT* qg = static_cast<const QT*>(a.q) + ((int64_t)s * a.num_heads + (int64_t)kvh * G) * D;
  for (int i = lane; i < G * D; i += 64) q_s[i % D][i / D] = to_f32<QDT>(qg[i]);
  __syncthreads();

  const int t = lane & 15;
  const int c = lane >> 4;
  float m[G], lsum[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[h][j] = 0.f;
  }

  const KT* kc = static_cast<const KT*>(a.k) + (int64_t)kvh * D * BS;
  const KT* vc = static_cast<const KT*>(a.v) + (int64_t)kvh * D * BS;
  const int32_t* table = a.tables + (int64_t)s * a.max_blocks;

  // Ring of raw K/V registers, kDepth blocks deep, for small groups (q of the
  // lane's D/4 rows for all G heads then fits in registers as well: the QK
  // loop is unrolled and reads the ring at fixed indices). Larger groups keep
  // one block at a time, its id read at the step and K and V loaded inside
  // it, as the ring would cost their occupancy.
  typedef typename Row16<KDT>::raw_t vraw_t;
  constexpr bool kRing = G * D / 4 <= 32;
  constexpr int kSlotRegs = D / 4 + DPL * 4 * Row16<KDT>::kPieces;
  constexpr int kDepth = !kRing ? 1 : (kSlotRegs <= 32 ? 4 : 2);
  KT kraw[kRing ? kDepth : 1][kRing ? D / 4 : 1];
  vraw_t vraw[kRing ? kDepth : 1][kRing ? DPL : 1];
  int64_t phys_of[kDepth];

  const int b0 = tok0 / BS;                        // tok0 is a multiple of the block size
  const int nblk = (tok1 - tok0 + BS - 1) / BS;    // 0 for an empty sequence
  int ids = 0;                                     // physical id of block (64-block chunk) + lane
  auto issue = [&](const int j, const int slot) __attribute__((always_inline)) {
    if constexpr (!kRing) {
      phys_of[slot] = clamp_block(a, table[b0 + j]);   // wave-uniform: a scalar load
      return;
    }
    if ((j & 63) == 0) {
      const int jj = j + lane;
      ids = jj < nblk ? (int)clamp_block(a, table[b0 + jj]) : 0;
    }
    phys_of[slot] = __builtin_amdgcn_readlane(ids, j & 63);
    {
      const KT* kb = kc + phys_of[slot] * a.block_stride;
      const KT* vb = vc + phys_of[slot] * a.block_stride;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) kraw[slot][i] = kb[(4 * i + c) * BS + t];
#pragma unroll
      for (int jr = 0; jr < DPL; ++jr) Row16<KDT>::load(vb + (lane + 64 * jr) * BS, vraw[slot][jr]);
    }
  };

  auto compute = [&](const int j, const int slot) __attribute__((always_inline)) {
    const int nvalid = min(BS, tok1 - (b0 + j) * BS);
    const KT* kb = kc + phys_of[slot] * a.block_stride;
    const KT* vb = vc + phys_of[slot] * a.block_stride;

    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    if constexpr (kRing) {
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const int d = 4 * i + c;
        const float kv = to_f32<KDT>(kraw[slot][i]);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(q_s[d][h], kv, acc[h]);
      }
    } else {
#pragma unroll 8
      for (int i = 0; i < D / 4; ++i) {
        const int d = 4 * i + c;
        const float kv = to_f32<KDT>(kb[d * BS + t]);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(q_s[d][h], kv, acc[h]);
      }
    }

    const bool valid = t < nvalid;
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = acc[h];
      x += shfl_xor_f32(x, 16);
      x += shfl_xor_f32(x, 32);
      const float sc = valid ? x * a.score_scale : -INFINITY;
      float mx = sc;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, shfl_xor_f32(mx, off));
      const float m_new = fmaxf(m[h], mx);
      alpha[h] = exp2f(m[h] - m_new);
      const float p = valid ? exp2f(sc - m_new) : 0.f;
      float ps = p;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ps += shfl_xor_f32(ps, off);
      lsum[h] = lsum[h] * alpha[h] + ps;
      m[h] = m_new;
      if (c == 0) p_s[h][t] = p;
    }
    __syncthreads();

#pragma unroll
    for (int jr = 0; jr < DPL; ++jr) {
      float vv[16];
      if constexpr (kRing) {
        Row16<KDT>::widen(vraw[slot][jr], vv);
      } else {
        vraw_t x;
        Row16<KDT>::load(vb + (lane + 64 * jr) * BS, x);
        Row16<KDT>::widen(x, vv);
      }
#pragma unroll
      for (int tt = 0; tt < BS; ++tt) vv[tt] = tt < nvalid ? vv[tt] : 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float pv = 0.f;
#pragma unroll
        for (int tt = 0; tt < BS; ++tt) pv = fmaf(p_s[h][tt], vv[tt], pv);
        o[h][jr] = o[h][jr] * alpha[h] + pv;
      }
    }
    __syncthreads();
  };

  // Block j + kDepth - 1 goes into the slot block j - 1 has released.
  static_for<kDepth - 1>([&](auto J) __attribute__((always_inline)) {
    if (J() < nblk) issue(J(), J());
  });
  if constexpr (kRing) {
    for (int jb = 0; jb < nblk; jb += kDepth) {
      static_for<kDepth>([&](auto SL) __attribute__((always_inline)) {
        const int j = jb + SL();
        if (j < nblk) {
          if (j + kDepth - 1 < nblk) issue(j + kDepth - 1, (SL() + kDepth - 1) % kDepth);
          compute(j, SL());
        }
      });
    }
  } else {
    for (int j = 0; j < nblk; ++j) {
      issue(j, 0);
      compute(j, 0);
    }
  }

  if (nparts == 1) {
    const int64_t obase = ((int64_t)s * a.num_heads + (int64_t)kvh * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = lsum[h] > 0.f ? a.v_scale / lsum[h] : 0.f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) store_out<QDT>(a.out, obase + (int64_t)h * D + lane + 64 * j, o[h][j] * inv);
    }
  } else {
    const int64_t slot = ((int64_t)s * a.num_kv_heads + kvh) * a.max_parts + part;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int j = 0; j < DPL; ++j) a.part_o[(slot * G + h) * D + lane + 64 * j] = o[h][j] * a.v_scale;
      if (lane == 0) {
        a.part_m[slot * G + h] = m[h];
        a.part_l[slot * G + h] = lsum[h];
      }
    }
  }
}

template <int QDT, int KDT, int D>
hipError_t launch_g(const Args& a, int group, dim3 grid, hipStream_t st) {
  switch (group) {
    case 1: valu_partition_kernel<QDT, KDT, D, 1><<<grid, 64, 0, st>>>(a); break;
    case 2: valu_partition_kernel<QDT, KDT, D, 2><<<grid, 64, 0, st>>>(a); break;
    case 4: valu_partition_kernel<QDT, KDT, D, 4><<<grid, 64, 0, st>>>(a); break;
    case 8: valu_partition_kernel<QDT, KDT, D, 8><<<grid, 64, 0, st>>>(a); break;
    case 16: valu_partition_kernel<QDT, KDT, D, 16><<<grid, 64, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QDT, int KDT>
hipError_t launch_d(const Args& a, int head_dim, int group, dim3 grid, hipStream_t st) {
  if (head_dim == 64) return launch_g<QDT, KDT, 64>(a, group, grid, st);
  if (head_dim == 128) return launch_g<QDT, KDT, 128>(a, group, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

bool valu_supported(int q_dtype, int kv_dtype, int head_dim, int group) {
  const bool types = (q_dtype == kF32 && kv_dtype == kF32) || (q_dtype == kBF16 && kv_dtype == kBF16) ||
                     (q_dtype == kBF16 && kv_dtype == kE5M2) || (q_dtype == kBF16 && kv_dtype == kE4M3);
  const bool dims = head_dim == 64 || head_dim == 128;
  const bool g = group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
  return types && dims && g;
}

hipError_t launch_valu(const Args& a, int q_dtype, int kv_dtype, int head_dim, int group,
                       hipStream_t stream) {
  const dim3 grid = partition_grid(a);
  if (q_dtype == kF32 && kv_dtype == kF32) return launch_d<kF32, kF32>(a, head_dim, group, grid, stream);
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_d<kBF16, kBF16>(a, head_dim, group, grid, stream);
  if (q_dtype == kBF16 && kv_dtype == kE5M2) return launch_d<kBF16, kE5M2>(a, head_dim, group, grid, stream);
  if (q_dtype == kBF16 && kv_dtype == kE4M3) return launch_d<kBF16, kE4M3>(a, head_dim, group, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
