// HIP kernels of the paged KV-cache path for gfx950 (CDNA4, wave64).
//
//  * kv write      : scatter of new tokens' K/V granules to their slots
//                    (vLLM 技术内幕, section 2.1: reshape_and_cache).
//  * block copy    : copy-on-write data move (juhe.plus, section 3.8).
//  * decode        : split-K over 256-token partitions of each sequence;
//                    each wave walks its partition's blocks through the
//                    block table (juhe.plus, section 3.6), keeps an online
//                    softmax and writes either the final row or a partial
//                    (max, sum, weighted V) that a merge pass combines.
//
// Pool layout (see pkv.h): pool[block][kv_head][K|V][tile]; a K tile is
// 16-byte granules of E consecutive d of one token, granule-major; a V tile
// is 16-byte granules of E consecutive tokens of one d.  With that layout a
// wave reads a K tile with lane = token (16 lanes x 16 B contiguous per
// granule) and a V tile with lane = d (64 lanes x 16 B contiguous), both as
// whole 16-byte loads, so no transpose through LDS is needed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

constexpr int BS = kBlockSize;
constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescale: the running max is only raised when a new score exceeds it
// by more than this (log2 units), so probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int ES>
__device__ __forceinline__ float granule_elem(const uint4& g, int e) {
  const uint32_t w[4] = {g.x, g.y, g.z, g.w};
  if constexpr (ES == 4) {
    return __uint_as_float(w[e]);
  } else {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
}

// ---- FP8 E4M3 (OCP): encode with round to nearest even, saturating
// magnitudes above 448 to 448; `sign` supplies the sign bit (0 or 0x80).
__device__ __forceinline__ uint32_t e4m3_code(float y, uint32_t sign) {
  const uint32_t au = __float_as_uint(y) & 0x7FFFFFFFu;
  if (au > 0x7F800000u) return sign | 0x7Fu;           // NaN
  const float a = __uint_as_float(au);
  if (a >= 448.f) return sign | 0x7Eu;                 // saturate (infinities too)
  if (a < 0.015625f)                                   // below 2^-6: steps of 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.f);  // 0..8 (8 = smallest normal)
  const uint32_t e = (au >> 23) - 120u;                // E4M3 biased exponent, 1..15
  uint32_t m = (au >> 20) & 7u;
  const uint32_t rest = au & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;  // a carry bumps e
  return sign | ((e << 3) + m);
}

typedef float f32x2v_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// Two E4M3 codes (bytes 2 HI, 2 HI + 1 of w) -> two floats / two bf16.
template <bool HI>
__device__ __forceinline__ f32x2v_t fp8x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_f16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// K/V bytes that a call reads once (decode rows, multi-query rows, the V
// conversion pass) are loaded non-temporally: the caches treat them as a
// stream and do not keep them at the expense of other lines.  On the 8B GQA
// decode batch this took the call from 0.268-0.270 to 0.245-0.247 ms (bf16)
// and from 0.160 to 0.146 ms (FP8 cache).  The prefill tiles' copies keep the
// default policy: every q tile of a kv head re-reads that head's K/V.
typedef unsigned int u32x4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once(const char* p) {
  const u32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Max / sum over the 64 lanes of the wave; every lane gets the same value.
// Rows of 16 lanes are reduced with DPP (quad swaps, half-row and row
// mirrors), then the four row results are combined.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform64(long long v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Orders one wave's LDS writes before its later LDS reads by other lanes.
// A wave's LDS operations execute in issue order, so keeping the compiler
// from moving accesses across this point is enough; waves of a workgroup
// that work independently need no workgroup barrier.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// KV write: one thread per (token, kv head, 16-byte granule of the row).
// ---------------------------------------------------------------------------
template <int ES>
__global__ __launch_bounds__(256) void k_kv_write(char* __restrict__ kv, size_t block_bytes,
                                                  int hkv, int D, const uint4* __restrict__ k_new,
                                                  const uint4* __restrict__ v_new,
                                                  const int64_t* __restrict__ slots, int64_t total) {
  constexpr int E = 16 / ES;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int KG = D / E;
  const int c = (int)(i % KG);
  const int64_t r = i / KG;
  const int h = (int)(r % hkv);
  const int64_t t = r / hkv;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  char* head = kv + blk * (int64_t)block_bytes + (int64_t)h * (2 * BS * D * ES);
  // K: the granule keeps its 16 bytes; it moves to granule index c * BS + off.
  *reinterpret_cast<uint4*>(head + (c * BS + off) * 16) = k_new[i];
  // V: element d = c * E + e of token off goes to ((off / E) * D + d) * E + off % E.
  const uint4 g = v_new[i];
  char* vt = head + BS * D * ES;
  const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = c * E + e;
    const int64_t el = ((int64_t)(off / E) * D + d) * E + (off % E);
    if constexpr (ES == 4) {
      reinterpret_cast<uint32_t*>(vt)[el] = w[e];
    } else {
      reinterpret_cast<uint16_t*>(vt)[el] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
    }
  }
}

// FP8 cache: one thread per (token, kv head, 16 consecutive d).  It reads the
// 16 bf16 inputs of K and of V, quantizes them (x * (1 / scale) in float32,
// then the nearest E4M3 code) and writes one 16-byte K granule and 16 bytes
// of the V tile (one per d, at the token's offset in that d's granule).
__global__ __launch_bounds__(256) void k_kv_write_fp8(char* __restrict__ kv, size_t block_bytes,
                                                      int hkv, int D,
                                                      const uint4* __restrict__ k_new,
                                                      const uint4* __restrict__ v_new,
                                                      const int64_t* __restrict__ slots,
                                                      int64_t total, float k_inv, float v_inv) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int KG = D / 16;
  const int c = (int)(i % KG);
  const int64_t r = i / KG;            // row (token, kv head)
  const int h = (int)(r % hkv);
  const int64_t t = r / hkv;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  char* head = kv + blk * (int64_t)block_bytes + (int64_t)h * (2 * BS * D);
  auto quantize16 = [](const uint4* src, float inv, uint32_t (&out)[4]) {
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t bits = (w[(4 * q + e) >> 1] >> (((4 * q + e) & 1) * 16)) & 0xFFFFu;
        const float x = __uint_as_float(bits << 16);
        word |= e4m3_code(x * inv, (bits >> 8) & 0x80u) << (8 * e);
      }
      out[q] = word;
    }
  };
  const int64_t src = r * (D / 8) + 2 * c;  // 16 bf16 = two uint4
  uint32_t kq[4], vq[4];
  quantize16(k_new + src, k_inv, kq);
  quantize16(v_new + src, v_inv, vq);
  // K: granule c of token `off` sits at (c * BS + off) * 16
  *reinterpret_cast<uint4*>(head + (c * BS + off) * 16) = make_uint4(kq[0], kq[1], kq[2], kq[3]);
  // V: element (off, d) at d * 16 + off (one 16-token granule per d)
  unsigned char* vt = reinterpret_cast<unsigned char*>(head + BS * D);
#pragma unroll
  for (int e = 0; e < 16; ++e) vt[(c * 16 + e) * 16 + off] = (unsigned char)(vq[e >> 2] >> (8 * (e & 3)));
}

hipError_t launch_kv_write(const CacheDesc& c, const void* k_new, const void* v_new,
                           const int64_t* slots, int64_t num_tokens, hipStream_t stream) {
  if (c.fp8) {
    const int64_t total = num_tokens * c.hkv * (c.head_size / 16);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_kv_write_fp8, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       c.kv, c.block_bytes, c.hkv, c.head_size, (const uint4*)k_new,
                       (const uint4*)v_new, slots, total, c.k_inv, c.v_inv);
    return hipGetLastError();
  }
  const int64_t total = num_tokens * c.hkv * (c.head_size * c.dtype_bytes / 16);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (c.dtype_bytes == 4)
    hipLaunchKernelGGL(k_kv_write<4>, grid, dim3(256), 0, stream, c.kv, c.block_bytes, c.hkv,
                       c.head_size, (const uint4*)k_new, (const uint4*)v_new, slots, total);
  else
    hipLaunchKernelGGL(k_kv_write<2>, grid, dim3(256), 0, stream, c.kv, c.block_bytes, c.hkv,
                       c.head_size, (const uint4*)k_new, (const uint4*)v_new, slots, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block copy: one thread per 16-byte granule of each (src, dst) pair.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_block_copy(char* __restrict__ kv, int64_t granules_per_block,
                                                    const int64_t* __restrict__ pairs, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t pr = i / granules_per_block;
  const int64_t g = i % granules_per_block;
  const int64_t src = pairs[2 * pr];
  const int64_t dst = pairs[2 * pr + 1];
  const uint4* s = reinterpret_cast<const uint4*>(kv) + src * granules_per_block + g;
  uint4* d = reinterpret_cast<uint4*>(kv) + dst * granules_per_block + g;
  *d = *s;
}

hipError_t launch_block_copy(const CacheDesc& c, const int64_t* pairs, int64_t num_pairs,
                             hipStream_t stream) {
  const int64_t gpb = (int64_t)(c.block_bytes / 16);
  const int64_t total = gpb * num_pairs;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_block_copy, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     c.kv, gpb, pairs, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block swap: the same granule copy with one side in host memory the GPU
// reaches through its device mapping (every access crosses the host link;
// each wave moves 1 KiB per instruction, and many waves keep the link busy).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_block_swap(const char* __restrict__ src_base,
                                                    char* __restrict__ dst_base,
                                                    int64_t granules_per_block,
                                                    const int64_t* __restrict__ pairs,
                                                    int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t pr = i / granules_per_block;
  const int64_t g = i % granules_per_block;
  const uint4* s = reinterpret_cast<const uint4*>(src_base) + pairs[2 * pr] * granules_per_block + g;
  uint4* d = reinterpret_cast<uint4*>(dst_base) + pairs[2 * pr + 1] * granules_per_block + g;
  *d = *s;
}

hipError_t launch_block_swap(const CacheDesc& c, char* host_dev_ptr, const int64_t* pairs,
                             int64_t num_pairs, bool to_host, hipStream_t stream) {
  const int64_t gpb = (int64_t)(c.block_bytes / 16);
  const int64_t total = gpb * num_pairs;
  if (total == 0) return hipSuccess;
  const char* src = to_host ? c.kv : host_dev_ptr;
  char* dst = to_host ? host_dev_ptr : c.kv;
  hipLaunchKernelGGL(k_block_swap, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     src, dst, gpb, pairs, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Read probe: the decode's access pattern without its arithmetic.  Wave w
// reads slices [w n / W, (w + 1) n / W) of the list (each the K and V tiles of
// one (block, kv head), 1 KiB per instruction, non-temporal like the decode's
// loads), two slices per step with the next step's loads in flight, and
// writes the XOR of every 32-bit word it read.  Slice ids come 64 at a time
// in one vector load, the next 64 requested with the current ones' first
// step.
// ---------------------------------------------------------------------------
template <int NLD>  // 16-byte loads per lane and slice
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_read_slices(
    const char* __restrict__ kv, size_t block_bytes, int hkv, const int64_t* __restrict__ slices,
    int64_t n, int waves, uint32_t* __restrict__ sink) {
  constexpr int SLICE = NLD * 1024;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x;
  const int64_t a = (int64_t)w * n / waves, b = (int64_t)(w + 1) * n / waves;
  uint32_t x = 0;
  if (a < b) {
    const int64_t cnt = b - a;
    const int64_t steps = (cnt + 1) / 2;
    int64_t ids = slices[min(a + lane, b - 1)];
    int64_t ids_next = slices[min(a + 64 + lane, b - 1)];
    auto base_of = [&](int64_t k) -> const char* {  // slice a + k (k < cnt), from the id registers
      const int64_t sl = uniform64(__shfl(ids, (int)(k & 63)));
      return kv + (size_t)(sl / hkv) * block_bytes + (size_t)(sl % hkv) * SLICE + lane * 16;
    };
    auto load_step = [&](uint4 (&r)[2 * NLD], int64_t k) {
      const char* p0 = base_of(2 * k);
      const char* p1 = 2 * k + 1 < cnt ? base_of(2 * k + 1) : p0;
#pragma unroll
      for (int i = 0; i < NLD; ++i) r[i] = load_once(p0 + i * 1024);
      if (2 * k + 1 < cnt) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) r[NLD + i] = load_once(p1 + i * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < NLD; ++i) r[NLD + i] = make_uint4(0, 0, 0, 0);
      }
    };
    auto fold = [&](const uint4 (&r)[2 * NLD]) {
#pragma unroll
      for (int i = 0; i < 2 * NLD; ++i) x ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    };
    // ids of slices a + 64 c .. are in `ids` while steps 32 c .. 32 c + 31 load
    auto advance_ids = [&](int64_t k) {  // before loading step k
      if (k > 0 && (k & 31) == 0) {
        ids = ids_next;
        ids_next = slices[min(a + 64 * (k / 32 + 1) + lane, b - 1)];
      }
    };
    uint4 ra[2 * NLD], rb[2 * NLD];
    load_step(ra, 0);
    for (int64_t k = 0; k < steps; k += 2) {
      if (k + 1 < steps) {
        advance_ids(k + 1);
        load_step(rb, k + 1);
      }
      fold(ra);
      if (k + 1 >= steps) break;
      if (k + 2 < steps) {
        advance_ids(k + 2);
        load_step(ra, k + 2);
      }
      fold(rb);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  if (lane == 0) sink[w] = x;
}

hipError_t launch_read_slices(const CacheDesc& c, const int64_t* slices, int64_t n, int waves,
                              uint32_t* sink, hipStream_t stream) {
  const size_t slice = (size_t)2 * BS * c.head_size * c.dtype_bytes;
  const dim3 grid((unsigned)waves);
  switch (slice / 1024) {
    case 2: hipLaunchKernelGGL(k_read_slices<2>, grid, dim3(64), 0, stream, c.kv, c.block_bytes, c.hkv, slices, n, waves, sink); break;
    case 4: hipLaunchKernelGGL(k_read_slices<4>, grid, dim3(64), 0, stream, c.kv, c.block_bytes, c.hkv, slices, n, waves, sink); break;
    case 8: hipLaunchKernelGGL(k_read_slices<8>, grid, dim3(64), 0, stream, c.kv, c.block_bytes, c.hkv, slices, n, waves, sink); break;
    case 16: hipLaunchKernelGGL(k_read_slices<16>, grid, dim3(64), 0, stream, c.kv, c.block_bytes, c.hkv, slices, n, waves, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode work units.  A unit is one partition of one decode row: a full
// 256-token partition, or the shorter last partition of a row.  All full
// units come first (sequence by sequence), then the partial ones from the
// longest size class to the shortest, so the short work lands at the end of
// the grid and evens out the tail.  A wave finds its unit's sequence with a
// scan over the lengths.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int row_len(const int32_t* seq_lens, const int32_t* qsl, int s) {
  const int ql = qsl ? qsl[s + 1] - qsl[s] : 1;
  return ql == 1 ? seq_lens[s] : 0;  // only single-query rows are decode rows
}
struct FullUnits {
  __device__ int operator()(int L) const { return L > 0 ? L / kPartTokens : 0; }
};
// The short last partitions are numbered by size class: class k holds the
// rows whose last partition takes 8 - k steps of 32 tokens, so larger ones
// are handed out first.
__device__ __forceinline__ int partial_class(int L) {
  const int rem = L % kPartTokens;
  return rem ? kPartTokens / 32 - (rem + 31) / 32 : -1;
}
struct PartialClass {
  int k;
  __device__ int operator()(int L) const { return (L > 0 && partial_class(L) == k) ? 1 : 0; }
};

// Sum over sequences [0, s_end) of count(row length); every lane gets it.
template <typename F>
__device__ int units_before(const int32_t* seq_lens, const int32_t* qsl, int s_end, F count) {
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int s0 = 0; s0 < s_end; s0 += 256) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = s0 + 4 * lane + k;
      acc += (s < s_end) ? count(row_len(seq_lens, qsl, s)) : 0;
    }
  }
  return (int)wave_sum((float)acc);  // exact: counts stay far below 2^24
}

// Find the sequence holding item u when sequence s has count(L_s) items,
// and u's index among them.  Each lane counts 4 consecutive sequences, so
// 256 lengths are read with four independent loads per lane before one wave
// scan.  Returns the sequence's length in len_out.
template <typename F>
__device__ bool find_unit(int u, const int32_t* seq_lens, const int32_t* qsl, int num_seqs, F count,
                          int& s_out, int& idx_out, int& len_out) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int s0 = 0; s0 < num_seqs; s0 += 256) {
    int n[4], len[4];
    int tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = s0 + 4 * lane + k;
      len[k] = (s < num_seqs) ? row_len(seq_lens, qsl, s) : 0;
      n[k] = count(len[k]);
      tot += n[k];
    }
    int incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int total = __shfl(incl, 63);
    if (u < base + total) {
      const unsigned long long m = __ballot(base + incl > u);
      const int hit = __ffsll((unsigned long long)m) - 1;
      // inside the lane that holds u: the first of its 4 sequences whose
      // range ends past u
      const int run = base + incl - tot;
      int kk = 3, before = run, start = run;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (kk == 3 && u < start + n[k]) { kk = k; before = start; }
        start += n[k];
      }
      if (!(u < before + n[kk])) before = run + n[0] + n[1] + n[2];
      int lk = len[0];
#pragma unroll
      for (int k = 1; k < 4; ++k) lk = (kk == k) ? len[k] : lk;
      s_out = uniform(__shfl(s0 + 4 * lane + kk, hit));
      idx_out = uniform(__shfl(u - before, hit));
      len_out = uniform(__shfl(lk, hit));
      return true;
    }
    base += total;
  }
  return false;
}

// ---------------------------------------------------------------------------
// Decode partition pass.  One wave per (unit, kv head); the wave serves all
// G query heads that share the kv head, so each K/V byte is read once.
// A step covers 2 blocks = 32 tokens:
//   K: lanes 2t and 2t+1 of each 32-lane half hold the two halves of token
//      t's K row; per-lane partial dot products with q (broadcast from LDS)
//      are completed by one DPP add with the neighbour lane.
//   softmax: wave max per head; the running max only moves when exceeded by
//      kRescaleSlack, and then acc and the sums are rescaled.
//   V: lane = d (D/64 values per lane); probabilities come from LDS.
// Loads of step i+1 are issued before step i is computed.
// ---------------------------------------------------------------------------
struct DecodeParams {
  const char* kv;
  size_t block_bytes;
  int hkv;
  const void* q;
  float* out;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int num_seqs;
  float scale_log2;
  float out_scale;  // multiplies every output (an fp8 cache's V scale)
  float* ws_acc;
  float* ws_ml;
  int full_units;   // units [0, full_units) are full partitions
  int total_items;  // units * kv heads
  int class_start[kPartClasses + 1];  // partial units before size class k
};

template <int ES, int D, int G, bool CHECK>
__device__ __forceinline__ void pv_block(const uint4 (&vr)[BS * D * ES / 16 / 64],
                                         const float* __restrict__ p_lds, int key_base,
                                         int valid_keys, float (&acc)[G][D / 64]) {
  constexpr int E = 16 / ES;
  constexpr int DPL = D / 64;
  // load i covers key granule i / DPL and the lane's d value i % DPL
#pragma unroll
  for (int kg = 0; kg < BS / E; ++kg) {
    float pk[E][G];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int g = 0; g < G; ++g) pk[e][g] = p_lds[(key_base + kg * E + e) * G + g];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) {
      const uint4 w = vr[kg * DPL + dd];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (CHECK && kg * E + e >= valid_keys) continue;
        const float v = granule_elem<ES>(w, e);
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g][dd] = fmaf(pk[e][g], v, acc[g][dd]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) asm volatile("" : "+v"(acc[g][dd]));
  }
}

// P.V over one block of an fp8 cache: vr[dd] holds the 16 keys' E4M3 codes
// of d = 64 dd + lane (one granule per d).  Codes become fp16 pairs (exact)
// and meet the probabilities, stored in LDS as fp16 [head][PS keys of the
// step], in v_dot2_f32_f16.  Keys at or past `valid_keys` get a zero value,
// so unwritten slots (any bits, NaN included) cannot reach the sums.
template <int D, int G, bool CHECK, int PS = 32>
__device__ __forceinline__ void pv_block_fp8(const uint4 (&vr)[D / 64], const uint16_t* __restrict__ p16,
                                             int key_base, int valid_keys, float (&acc)[G][D / 64]) {
  constexpr int DPL = D / 64;
  uint32_t pp[G][8];  // probability pairs (keys 2q, 2q + 1) of each head
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 a = *reinterpret_cast<const uint4*>(p16 + g * PS + key_base);
    const uint4 b = *reinterpret_cast<const uint4*>(p16 + g * PS + key_base + 8);
    pp[g][0] = a.x; pp[g][1] = a.y; pp[g][2] = a.z; pp[g][3] = a.w;
    pp[g][4] = b.x; pp[g][5] = b.y; pp[g][6] = b.z; pp[g][7] = b.w;
  }
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) {
    const uint32_t w[4] = {vr[dd].x, vr[dd].y, vr[dd].z, vr[dd].w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t v = (q & 1) ? fp8x2_f16<true>(w[q >> 1]) : fp8x2_f16<false>(w[q >> 1]);
      if (CHECK) {
        if (2 * q >= valid_keys) v = 0u;
        else if (2 * q + 1 >= valid_keys) v &= 0xFFFFu;
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[g][dd] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pp[g][q]),
                                            __builtin_bit_cast(f16x2_t, v), acc[g][dd], false);
    }
  }
}

template <int ES, int D>
struct DecodeShape {
  static constexpr int E = 16 / ES;                // elements per granule
  static constexpr int KG = D / E;                 // granules per K row
  static constexpr int KH = KG / 2;                // granules per lane (half row)
  static constexpr int VG = BS * D * ES / 16 / 64; // V granules per lane per block
  static constexpr int DPL = D / 64;               // d values per lane
  static constexpr int TILE = BS * D * ES;         // bytes of one K or V tile
  static constexpr int QES = ES == 4 ? 4 : 2;      // query element bytes (bf16 for fp8 caches)
  static constexpr int QKG = D * QES / 16;         // 16-byte granules per q row
  static constexpr int QKH = QKG / 2;              // per half row
  static constexpr int QROW = QKH * 16 + 16;       // LDS bytes of a padded half q row
};

template <int ES, int D>
struct StepRegs {
  uint4 k[DecodeShape<ES, D>::KH];
  uint4 v[2][DecodeShape<ES, D>::VG];
};

// Steps of the stream decode.  A wave's rate grows with the bytes of one
// step more than with the number of waves holding steps in flight: on the
// 8B GQA batch, one bf16 wave per SIMD (16 KiB steps) streamed 4.93 TB/s
// where two FP8 waves per SIMD with 8 KiB steps reached 4.00 and three 4.48.
// So an FP8 step covers four blocks (16 KiB of K and V at D = 128) and each
// lane takes one token's whole K row.  bf16 with one query head per kv head
// takes four-block steps too (32 KiB at D = 128, one wave per SIMD: 13B
// shape 0.805-0.810 of 8 TB/s against 0.795-0.798, 7B 0.713-0.714 against
// 0.710-0.712); with more heads per kv head one wave cannot overlap their
// arithmetic with its loads (8B GQA: 0.64 against 0.68), so those and fp32
// keep two blocks per step, each lane half a K row.
template <int ES, int D, int G>
struct StreamShape {
  static constexpr int NB = ES == 1 || (ES == 2 && G == 1) ? 4 : 2;  // blocks per step
  static constexpr int STEP = NB * BS;                           // tokens per step
  static constexpr bool TPL = NB == 4;                           // one token per lane
  static constexpr int KL = TPL ? DecodeShape<ES, D>::KG         // K granules per lane
                                : DecodeShape<ES, D>::KH;
  static_assert(!TPL || STEP == 64, "one token per lane");
};
template <int ES, int D, int G>
struct StreamRegs {
  uint4 k[StreamShape<ES, D, G>::KL];
  uint4 v[StreamShape<ES, D, G>::NB][DecodeShape<ES, D>::VG];
};

// Per-item state of a decode wave: which unit of which row, and where.
struct DecodeItem {
  int valid;
  int s, part, L, row, kvh, unit;
  int tok0, tok_end, nsteps, nparts;
  int my_id;  // lane i < number of blocks of the unit: its i-th physical block
  int buf;    // which LDS q buffer holds this item's query rows
};

// LDS of one decode wave: two q buffers (each half row padded by 16 bytes so
// the two halves read in one instruction fall in different banks) and the
// probabilities of one step.
template <int ES, int D, int G>
struct DecodeLds {
  static constexpr int QBUF = G * 2 * DecodeShape<ES, D>::QROW;
  static constexpr int BYTES = 2 * QBUF + 32 * G * 4;
};

// One decode work item (unit, kv head) on one wave; `lds` is the wave's own
// DecodeLds area.  Waves are independent: only wave-level ordering is used.
template <int ES, int D, int G>
__device__ __forceinline__ void decode_item(const DecodeParams& p, int item, char* lds) {
  using S = DecodeShape<ES, D>;
  static_assert(D % 64 == 0, "head size must be a multiple of 64");
  static_assert(kPartTokens % 32 == 0 && kPartTokens / BS <= 64, "partition size");
  constexpr int QBUF = DecodeLds<ES, D, G>::QBUF;
  auto q_lds = [lds](int b) { return lds + b * QBUF; };
  float* p_lds = reinterpret_cast<float*>(lds + 2 * QBUF);

  const int lane = threadIdx.x & 63;
  const int hq = p.hkv * G;
  const int half = lane & 1;           // which half of the K row
  const int t_in_blk = (lane >> 1) & 15;
  const int bsel = lane >> 5;          // which block of the step
  const int k_lane_off = (half * S::KH * BS + t_in_blk) * 16;

  // Work item i = unit * hkv + kv head; this wave takes items
  // blockIdx.x, blockIdx.x + gridDim.x, ...  Units run full partitions first,
  // so the short last partitions fall at the end of every wave's list.
  auto setup = [&](DecodeItem& it, int item, int buf) {
    it.valid = item < p.total_items;
    if (!it.valid) return;
    it.kvh = item % p.hkv;
    it.unit = item / p.hkv;
    it.buf = buf;
    int s, part, L;
    if (it.unit < p.full_units) {
      find_unit(it.unit, p.seq_lens, p.qsl, p.num_seqs, FullUnits(), s, part, L);
    } else {
      const int v = it.unit - p.full_units;
      int k = 0;
#pragma unroll
      for (int c = 1; c < kPartClasses; ++c) k += v >= p.class_start[c] ? 1 : 0;
      find_unit(v - p.class_start[k], p.seq_lens, p.qsl, p.num_seqs, PartialClass{k}, s, part, L);
      part = L / kPartTokens;  // the last, partial partition of the row
    }
    it.s = s;
    it.part = part;
    it.L = L;
    it.nparts = (L + kPartTokens - 1) / kPartTokens;
    it.row = p.qsl ? p.qsl[s] : s;
    it.tok0 = part * kPartTokens;
    it.tok_end = min(L, it.tok0 + kPartTokens);
    const int nblk = (it.tok_end - it.tok0 + BS - 1) / BS;
    it.nsteps = (nblk + 1) / 2;
    // lane i < nblk holds the unit's i-th physical block id; later lanes
    // repeat the last one so over-reads stay inside valid blocks.
    const int32_t* bt = p.block_tables + (size_t)s * p.max_blocks + it.tok0 / BS;
    it.my_id = bt[min(lane, nblk - 1)];
    constexpr int QGR = G * S::KG;  // 16-byte granules of the group's q rows
    const uint4* src = reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) + ((size_t)it.row * hq + (size_t)it.kvh * G) * D * ES);
    for (int i = lane; i < QGR; i += 64) {
      const int g = i / S::KG, c = i % S::KG;
      const int hh = c / S::KH, cc = c % S::KH;
      *reinterpret_cast<uint4*>(q_lds(buf) + (g * 2 + hh) * S::QROW + cc * 16) = src[i];
    }
  };

  auto load = [&](StepRegs<ES, D>& r, const DecodeItem& it, int st) {
    const int b0 = uniform(__builtin_amdgcn_readlane(it.my_id, 2 * st));
    const int b1 = uniform(__builtin_amdgcn_readlane(it.my_id, 2 * st + 1));
    const char* head_base = p.kv + (size_t)it.kvh * 2 * S::TILE;
    const char* base0 = head_base + (size_t)b0 * p.block_bytes;
    const char* base1 = head_base + (size_t)b1 * p.block_bytes;
    const char* kp = (bsel ? base1 : base0) + k_lane_off;
#pragma unroll
    for (int c = 0; c < S::KH; ++c) r.k[c] = load_once(kp + c * BS * 16);
#pragma unroll
    for (int i = 0; i < S::VG; ++i) {
      r.v[0][i] = load_once(base0 + S::TILE + i * 1024 + lane * 16);
      r.v[1][i] = load_once(base1 + S::TILE + i * 1024 + lane * 16);
    }
  };

  float m_run[G], l_lane[G], acc[G][S::DPL];
  auto reset_state = [&]() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.f;
#pragma unroll
      for (int j = 0; j < S::DPL; ++j) acc[g][j] = 0.f;
    }
  };

  auto compute = [&](const StepRegs<ES, D>& r, const DecodeItem& it, int st) {
    // ---- scores: q granules are read from LDS one step ahead of use
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    const char* qh = q_lds(it.buf) + half * S::QROW;
    uint4 qcur[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qcur[g] = *reinterpret_cast<const uint4*>(qh + g * 2 * S::QROW);
#pragma unroll
    for (int c = 0; c < S::KH; ++c) {
      uint4 qnext[G];
      const int cn = c + 1 < S::KH ? c + 1 : c;
#pragma unroll
      for (int g = 0; g < G; ++g)
        qnext[g] = *reinterpret_cast<const uint4*>(qh + g * 2 * S::QROW + cn * 16);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 qg = qcur[g];
        const uint4 kg = r.k[c];
        if constexpr (ES == 2) {
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.x),
                                                  __builtin_bit_cast(bf16x2_t, kg.x), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.y),
                                                  __builtin_bit_cast(bf16x2_t, kg.y), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.z),
                                                  __builtin_bit_cast(bf16x2_t, kg.z), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.w),
                                                  __builtin_bit_cast(bf16x2_t, kg.w), sc[g], false);
        } else {
          sc[g] = fmaf(__uint_as_float(qg.x), __uint_as_float(kg.x), sc[g]);
          sc[g] = fmaf(__uint_as_float(qg.y), __uint_as_float(kg.y), sc[g]);
          sc[g] = fmaf(__uint_as_float(qg.z), __uint_as_float(kg.z), sc[g]);
          sc[g] = fmaf(__uint_as_float(qg.w), __uint_as_float(kg.w), sc[g]);
        }
        qcur[g] = qnext[g];
      }
      // Pin the partial sums here so the compiler cannot sink whole
      // dot products (keeping every q granule live) past this point.
#pragma unroll
      for (int g = 0; g < G; ++g) asm volatile("" : "+v"(sc[g]));
    }

    // ---- online softmax (log2 domain); the pair of lanes of a token
    // completes its dot product with one swap-add.
    const int tok = it.tok0 + st * 32 + (lane >> 1);
    const bool tok_ok = tok < it.tok_end;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float full = sc[g] + dpp_f<0xB1>(sc[g]);
      const float x = tok_ok ? full * p.scale_log2 : -INFINITY;
      const float mi = wave_max(x);
      if (mi > m_run[g] + kRescaleSlack) {
        const float corr = __builtin_amdgcn_exp2f(m_run[g] - mi);
        l_lane[g] *= corr;
#pragma unroll
        for (int j = 0; j < S::DPL; ++j) acc[g][j] *= corr;
        m_run[g] = mi;
      }
      const float pr = __builtin_amdgcn_exp2f(x - m_run[g]);
      if (half == 0) {
        l_lane[g] += pr;
        p_lds[(lane >> 1) * G + g] = pr;
      }
    }
    wave_sync();

    // ---- weighted V
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int valid = it.tok_end - (it.tok0 + (2 * st + j) * BS);
      if (valid >= BS)
        pv_block<ES, D, G, false>(r.v[j], p_lds, j * BS, BS, acc);
      else if (valid > 0)
        pv_block<ES, D, G, true>(r.v[j], p_lds, j * BS, valid, acc);
    }
    wave_sync();
  };

  auto finish = [&](const DecodeItem& it) {
    float l_tot[G];
#pragma unroll
    for (int g = 0; g < G; ++g) l_tot[g] = wave_sum(l_lane[g]);
    if (it.nparts == 1) {
      float* o = p.out + ((size_t)it.row * hq + (size_t)it.kvh * G) * D;
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int j = 0; j < S::DPL; ++j) o[g * D + j * 64 + lane] = acc[g][j] / l_tot[g];
      }
    } else {
      const size_t w = (size_t)it.unit * hq + (size_t)it.kvh * G;
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int j = 0; j < S::DPL; ++j) p.ws_acc[(w + g) * D + j * 64 + lane] = acc[g][j];
        if (lane == 0) {
          p.ws_ml[(w + g) * 2] = m_run[g];
          p.ws_ml[(w + g) * 2 + 1] = l_tot[g];
        }
      }
    }
    reset_state();
  };

  // The unit's steps, two register sets alternating: the loads of step
  // st + 1 are in flight while step st is computed.
  DecodeItem cur;
  setup(cur, item, 0);
  if (!cur.valid) return;
  reset_state();
  wave_sync();  // q rows visible
  StepRegs<ES, D> ra, rb;
  load(ra, cur, 0);
  for (int st = 0; st < cur.nsteps; st += 2) {
    if (st + 1 < cur.nsteps) load(rb, cur, st + 1);
    compute(ra, cur, st);
    if (st + 1 < cur.nsteps) {
      if (st + 2 < cur.nsteps) load(ra, cur, st + 2);
      compute(rb, cur, st + 1);
    }
  }
  finish(cur);
}

// Waves per SIMD the decode kernels are compiled for: two, except where
// their registers do not fit in half the register file (fp32 at D = 128 or
// G = 8; bf16 at D = 128 and G = 8, or G = 1 with its four-block steps; FP8
// at G = 8): those get one wave per SIMD and all 512 registers, so nothing
// spills to memory.
constexpr int decode_waves_per_simd(int es, int d, int g) {
  return (es == 4 && (d == 128 || g == 8)) || (es == 2 && d == 128 && (g == 8 || g == 1)) ||
                 (es == 1 && g == 8)
             ? 1
             : 2;
}

template <int ES, int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(
    decode_waves_per_simd(ES, D, G)))) void k_decode_partition(
    DecodeParams p) {
  __shared__ __align__(16) char lds[DecodeLds<ES, D, G>::BYTES];
  decode_item<ES, D, G>(p, blockIdx.x, lds);
}

// ---------------------------------------------------------------------------
// Merge pass for decode rows split over several partitions:
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// One workgroup per (sequence, kv head), one wave per query head of the
// group.  Lane p holds partition p's (m, l), so the max, the weights and the
// denominator are wave reductions; the weighted sum over partitions then
// runs with lanes over d and eight partitions' loads in flight at a time.
// Also writes the zero row of an empty sequence.
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(256) void k_decode_merge(DecodeParams p) {
  constexpr int DPL = D / 64;
  constexpr int NW = G < 4 ? G : 4;  // waves per workgroup
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (wave >= NW) return;
  const int kvh = blockIdx.x % p.hkv;
  const int s = blockIdx.x / p.hkv;
  const int ql = p.qsl ? p.qsl[s + 1] - p.qsl[s] : 1;
  if (ql != 1) return;
  const int L = p.seq_lens[s];
  const int row = p.qsl ? p.qsl[s] : s;
  const int hq = p.hkv * G;
  if (L <= 0) {
    for (int g = wave; g < G; g += NW) {
      float* o = p.out + ((size_t)row * hq + (size_t)kvh * G + g) * D;
      for (int i = lane; i < D; i += 64) o[i] = 0.f;
    }
    return;
  }
  const int nparts = (L + kPartTokens - 1) / kPartTokens;
  if (nparts == 1) return;
  // partition q < nfull is unit u_full + q; a partial last one is unit u_part
  const int nfull = L / kPartTokens;
  const int u_full = units_before(p.seq_lens, p.qsl, s, FullUnits());
  const int kc = partial_class(L);
  const int u_part =
      kc < 0 ? 0 : p.full_units + p.class_start[kc] + units_before(p.seq_lens, p.qsl, s, PartialClass{kc});
  auto unit_of = [&](int q) { return q < nfull ? u_full + q : u_part; };
  for (int g = wave; g < G; g += NW) {
    const size_t gh = (size_t)kvh * G + g;
    float M = -INFINITY;
    for (int c = 0; c < nparts; c += 64) {
      const int q = c + lane;
      if (q < nparts) M = fmaxf(M, p.ws_ml[((size_t)unit_of(q) * hq + gh) * 2]);
    }
    M = wave_max(M);
    float den = 0.f;
    float num[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) num[j] = 0.f;
    for (int c = 0; c < nparts; c += 64) {
      const int q = c + lane;
      float wq = 0.f;
      if (q < nparts) {
        const size_t wi = (size_t)unit_of(q) * hq + gh;
        wq = __builtin_amdgcn_exp2f(p.ws_ml[wi * 2] - M);
        den = fmaf(wq, p.ws_ml[wi * 2 + 1], den);
      }
      const int n = min(64, nparts - c);
      int i = 0;
      for (; i + 8 <= n; i += 8) {
        float a[8][DPL];
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int j = 0; j < DPL; ++j)
            a[k][j] = p.ws_acc[((size_t)unit_of(c + i + k) * hq + gh) * D + j * 64 + lane];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), i + k));
#pragma unroll
          for (int j = 0; j < DPL; ++j) num[j] = fmaf(wk, a[k][j], num[j]);
        }
      }
      for (; i < n; ++i) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), i));
#pragma unroll
        for (int j = 0; j < DPL; ++j)
          num[j] = fmaf(wk, p.ws_acc[((size_t)unit_of(c + i) * hq + gh) * D + j * 64 + lane], num[j]);
      }
    }
    den = wave_sum(den);
    float* o = p.out + ((size_t)row * hq + (size_t)kvh * G + g) * D;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j * 64 + lane] = num[j] / den;
  }
}

// ---------------------------------------------------------------------------
// Stream decode (calls without prefill rows).  The decode work is laid out
// on one line of cost: item (row s, kv head h), h fastest, costs a setup
// charge c0 followed by one unit per step of the row (32 or 64 tokens, see
// StreamShape).  The line is
// cut into `waves` equal ranges, one per wave, and the grid is sized to the
// waves the GPU holds at once, so every wave streams the same number of
// steps and all finish together: there is no tail of short units.
//
// A wave walks its range step by step.  Its pipeline runs two steps ahead:
// while step k is computed the K/V of step k + 1 are in flight, and the
// block ids of step k + 2 travel in one small vector load issued with them
// (as do the q rows of an item that starts at step k + 1), so waiting for a
// step's data also covers its metadata and item changes cost no bubble.
//
// An item whose steps fall in one wave's range is finished there.  An item
// split over waves wA..wB leaves one partial (max, sum, weighted V) per wave
// in the workspace; each contributor then counts itself in the item's
// counter, and the last one merges the partials into the output row, so no
// second launch is needed.  Counters carry the call's epoch in their upper
// half: a counter whose epoch differs is stale and counts as zero, so the
// workspace needs no clearing between calls.  The merging wave puts its
// counter back to 0 (epochs are odd, so 0 is never current): a graph that
// replays a captured call, epoch and all, then starts every replay from
// stale counters too.
// ---------------------------------------------------------------------------
// Partials travel between waves that may sit on different XCDs, whose L2
// caches are not coherent with each other.  They are written and read with
// agent-scope relaxed atomics (coherent at the device level, instruction by
// instruction); a writer waits until its stores are complete before it
// counts itself in, and the merging wave reads the partials only after its
// count, so no fence has to write back or invalidate a whole L2.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct StreamParams {
  DecodeParams d;
  int waves;                     // ranges = grid size
  int c0;                        // setup charge per item, in steps
  unsigned epoch;                // distinct per call
  int rounds;                    // > 1: waves per SIMD, which rotate their issue priority
  // Share of the cost line per wave, in units of 1/1024 of an equal share:
  // waves below `half` weigh wt[0] (even w) or wt[1] (odd w), the others
  // wt[2] or wt[3].  Equal shares: all 1024 and half = waves.  Otherwise
  // half = waves / 2, a multiple of 2, and the four sum to 4096.
  int wt[4];
  int half;
  unsigned long long* counters;  // [num_seqs][hkv]
  float* part_acc;               // [2 * waves][G][D]
  float* part_ml;                // [2 * waves][G][2]
};

// One (item, step) position of a wave's walk.  All fields are wave-uniform.
struct StreamCur {
  int valid;
  int s, h, j;  // sequence, kv head, step within the item
  int n, L;     // steps and tokens of the sequence
  int row;      // output row of the sequence
  long long A;  // cost position of step 0 of the item
};

// How the cost line is cut into wave ranges in one call: `waves` ranges,
// wave w weighing wt[w < half ? 0 : 2] (even w) or wt[... + 1] (odd w), in
// units of 1/1024 of an equal share.
struct StreamSplit {
  int waves, half;
  int wt[4];
};
// Every wave computes the same split from the device total T: the host's
// weights, unless T is below two units per wave (a call replayed from a
// graph after the lengths shrank); then max(1, T / 2) waves with equal
// shares.  Either way every range holds at least one unit (weights stay
// within half and twice an equal share), so the waves between the first and
// the last contributor of an item all contribute to it.
__device__ __forceinline__ StreamSplit stream_split(const StreamParams& sp, long long T) {
  StreamSplit r;
  r.waves = sp.waves;
  r.half = sp.half;
  for (int k = 0; k < 4; ++k) r.wt[k] = sp.wt[k];
  if (T < 2LL * sp.waves) {
    r.waves = (int)max(1LL, T / 2);
    r.half = r.waves;
    for (int k = 0; k < 4; ++k) r.wt[k] = 1024;
  }
  return r;
}
// Weighted position where the range of wave w starts (the sum of the weights
// of waves 0 .. w - 1; waves * 1024 in all).
__device__ __forceinline__ long long stream_cum(const StreamSplit& sp, int w) {
  const int a = min(w, sp.half), b = w - a;
  return (long long)(a >> 1) * (sp.wt[0] + sp.wt[1]) + (a & 1) * sp.wt[0] +
         (long long)(b >> 1) * (sp.wt[2] + sp.wt[3]) + (b & 1) * sp.wt[2];
}
// First cost position of wave w's range (w = waves gives T).
__device__ __forceinline__ long long stream_start(const StreamSplit& sp, int w, long long T) {
  return T * stream_cum(sp, w) / ((long long)sp.waves * 1024);
}
// Wave whose range holds cost position t < T: the largest w with
// stream_start(w) <= t, i.e. the largest w with stream_cum(w) <= u, where u
// is the largest weighted position with floor(T u / (1024 waves)) <= t.
__device__ __forceinline__ int stream_wave_of(const StreamSplit& sp, long long t, long long T) {
  const long long u = ((t + 1) * (long long)sp.waves * 1024 - 1) / T;
  const long long c_half = stream_cum(sp, sp.half);
  int w;
  if (u < c_half) {
    const long long pr = u / (sp.wt[0] + sp.wt[1]);
    w = (int)(2 * pr + (u - pr * (sp.wt[0] + sp.wt[1]) >= sp.wt[0] ? 1 : 0));
  } else {
    const long long v = u - c_half;
    const long long pr = v / (sp.wt[2] + sp.wt[3]);
    w = sp.half + (int)(2 * pr + (v - pr * (sp.wt[2] + sp.wt[3]) >= sp.wt[2] ? 1 : 0));
  }
  return min(w, sp.waves - 1);
}

template <int ES, int D, int G>
struct StreamLds {
  static constexpr int QBUF = G * 2 * DecodeShape<ES, D>::QROW;
};

template <int ES, int D, int G>
__device__ __forceinline__ void stream_merge(const StreamParams& sp, int wA, int wB, float* o) {
  // o: the G output rows of the item (query heads kvh * G .. + G - 1)
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int nw = wB - wA + 1;
  auto slot_of = [wA](int w) { return 2 * w + (w == wA ? 1 : 0); };
  if (nw <= 8) {
    // every load first (contributors past nw repeat the last one and get
    // weight 0), then the arithmetic: one round trip to memory
    constexpr int K = 8;
    float m[G], l[G], a[G][K][DPL];
    const int my = slot_of(wA + min(lane, nw - 1));
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = load_agent(sp.part_ml + ((size_t)my * G + g) * 2);
      l[g] = load_agent(sp.part_ml + ((size_t)my * G + g) * 2 + 1);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int sk = slot_of(wA + min(k, nw - 1));
#pragma unroll
        for (int j = 0; j < DPL; ++j)
          a[g][k][j] = load_agent(sp.part_acc + ((size_t)sk * G + g) * D + j * 64 + lane);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float M = wave_max(lane < nw ? m[g] : -INFINITY);
      const float wq = lane < nw ? __builtin_amdgcn_exp2f(m[g] - M) : 0.f;
      const float den = wave_sum(wq * l[g]);
      float num[DPL];
#pragma unroll
      for (int j = 0; j < DPL; ++j) num[j] = 0.f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), k));
#pragma unroll
        for (int j = 0; j < DPL; ++j) num[j] = fmaf(wk, a[g][k][j], num[j]);
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[g * D + j * 64 + lane] = num[j] / den * sp.d.out_scale;
    }
    return;
  }
  for (int g = 0; g < G; ++g) {
    float M = -INFINITY;
    for (int c = 0; c < nw; c += 64) {
      const int w = wA + c + lane;
      if (c + lane < nw) {
        const int slot = 2 * w + (w == wA ? 1 : 0);
        M = fmaxf(M, load_agent(sp.part_ml + ((size_t)slot * G + g) * 2));
      }
    }
    M = wave_max(M);
    float den = 0.f, num[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) num[j] = 0.f;
    for (int c = 0; c < nw; c += 64) {
      const int w = wA + c + lane;
      float wq = 0.f;
      if (c + lane < nw) {
        const int slot = 2 * w + (w == wA ? 1 : 0);
        const float* ml = sp.part_ml + ((size_t)slot * G + g) * 2;
        wq = __builtin_amdgcn_exp2f(load_agent(ml) - M);
        den = fmaf(wq, load_agent(ml + 1), den);
      }
      const int n = min(64, nw - c);
      int i = 0;
      for (; i + 4 <= n; i += 4) {
        float a[4][DPL];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int w2 = wA + c + i + k;
          const int slot = 2 * w2 + (w2 == wA ? 1 : 0);
#pragma unroll
          for (int j = 0; j < DPL; ++j)
            a[k][j] = load_agent(sp.part_acc + ((size_t)slot * G + g) * D + j * 64 + lane);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), i + k));
#pragma unroll
          for (int j = 0; j < DPL; ++j) num[j] = fmaf(wk, a[k][j], num[j]);
        }
      }
      for (; i < n; ++i) {
        const int w2 = wA + c + i;
        const int slot = 2 * w2 + (w2 == wA ? 1 : 0);
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), i));
#pragma unroll
        for (int j = 0; j < DPL; ++j)
          num[j] = fmaf(wk, load_agent(sp.part_acc + ((size_t)slot * G + g) * D + j * 64 + lane), num[j]);
      }
    }
    den = wave_sum(den);
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[g * D + j * 64 + lane] = num[j] / den * sp.d.out_scale;
  }
}

template <int ES, int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(
    decode_waves_per_simd(ES, D, G)))) void k_decode_stream(StreamParams sp) {
  using S = DecodeShape<ES, D>;
  using SS = StreamShape<ES, D, G>;
  constexpr int QBUF = StreamLds<ES, D, G>::QBUF;
  constexpr int QGR = G * S::QKG;            // 16-byte granules of one item's q rows
  constexpr int NQ = (QGR + 63) / 64;        // per lane
  __shared__ __align__(16) char q_lds[QBUF];
  // one step's probabilities: fp32 [keys of the step][G], or (FP8) fp16
  // [G][64 keys]
  __shared__ __align__(16) float p_lds[SS::STEP * (ES == 1 ? 2 : 4) / 4 * G];
  __shared__ int len_lds[256];
  __shared__ int row_lds[256];

  const DecodeParams& p = sp.d;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x;
  const int W = sp.waves;
  const int hkv = p.hkv;
  const int hq = hkv * G;
  const int c0 = sp.c0;

  // Empty decode rows get zeros: sequences w, w + W, w + 2W, ...  Done at
  // the end of the wave's work, off the start-up chain of dependent loads.
  auto zero_rows = [&]() {
    for (long long sb = w; sb < p.num_seqs; sb += 64LL * W) {
      const long long s = sb + (long long)lane * W;
      bool zero = false;
      if (s < p.num_seqs) {
        const int ql = p.qsl ? p.qsl[s + 1] - p.qsl[s] : 1;
        zero = ql == 1 && p.seq_lens[s] <= 0;
      }
      unsigned long long m = __ballot(zero);
      while (m) {
        const int l = __ffsll(m) - 1;
        m &= m - 1;
        const long long sz = sb + (long long)l * W;
        const int row = p.qsl ? p.qsl[sz] : (int)sz;
        float* o = p.out + (size_t)row * hq * D;
        for (int i = lane; i < hq * D; i += 64) o[i] = 0.f;
      }
    }
  };

  // ---- the cost line, from the device lengths.  Lane l holds sequences
  // 4l .. 4l + 3 of every chunk of 256.  The host's copy of the lengths only
  // sized the grid: a call replayed from a captured graph after the lengths
  // have changed still covers every item (the grid and the workspace depend
  // on the wave count and the number of sequences, not on the lengths).
  auto cost_of = [&](int L) -> long long {
    return L > 0 ? (long long)hkv * ((L + SS::STEP - 1) / SS::STEP + c0) : 0;
  };
  struct ChunkCost {
    long long c[4], tot, incl;  // this lane's costs, their sum, inclusive scan over lanes
  };
  auto chunk_cost = [&](int first) {
    ChunkCost r;
    r.tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = first + 4 * lane + k;
      r.c[k] = cost_of(s < p.num_seqs ? row_len(p.seq_lens, p.qsl, s) : 0);
      r.tot += r.c[k];
    }
    r.incl = r.tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long t = __shfl_up(r.incl, off);
      if (lane >= off) r.incl += t;
    }
    return r;
  };
  const ChunkCost first = chunk_cost(0);
  const long long first_total = uniform64(__shfl(first.incl, 63));
  long long T = first_total;
  if (p.num_seqs > 256) {
    long long rest = 0;
    for (int sb = 256; sb < p.num_seqs; sb += 256) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int s = sb + 4 * lane + k;
        if (s < p.num_seqs) rest += cost_of(row_len(p.seq_lens, p.qsl, s));
      }
    }
    for (int off = 32; off > 0; off >>= 1) rest += __shfl_xor(rest, off);
    T += uniform64(rest);
  }
  const StreamSplit split = stream_split(sp, T);
  const long long cs = w < split.waves ? stream_start(split, w, T) : T;
  const long long ce = w < split.waves ? stream_start(split, w + 1, T) : T;
  if (cs >= ce) {
    zero_rows();
    return;
  }

  // ---- find the sequence whose cost range holds cs; keep its chunk of 256
  // decode lengths (and output rows) in LDS for the walk
  int s0 = 0;
  long long base = 0;  // cost before sequence s0
  auto load_chunk = [&](int first_seq) {
    for (int k = 0; k < 4; ++k) {
      const int s = first_seq + 4 * lane + k;
      len_lds[4 * lane + k] = s < p.num_seqs ? row_len(p.seq_lens, p.qsl, s) : 0;
      row_lds[4 * lane + k] = s < p.num_seqs ? (p.qsl ? p.qsl[s] : s) : 0;
    }
    wave_sync();
  };
  int s_found = -1;
  long long S_found = 0;
  auto pick = [&](const ChunkCost& cc) {  // cs lies in the chunk starting at s0
    const unsigned long long m = __ballot(base + cc.incl > cs);
    const int hit = __ffsll(m) - 1;
    long long start = base + cc.incl - cc.tot;  // cost before this lane's first sequence
    int kk = 3;
    long long Sk = start;
    bool found = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!found && cs < start + cc.c[k]) {
        kk = k;
        Sk = start;
        found = true;
      }
      start += cc.c[k];
    }
    s_found = uniform(__shfl(s0 + 4 * lane + kk, hit));
    S_found = uniform64(__shfl(Sk, hit));
  };
  if (cs < first_total) {
    pick(first);
  } else {
    base = first_total;
    for (s0 = 256; s0 < p.num_seqs; s0 += 256) {
      const ChunkCost cc = chunk_cost(s0);
      const long long total = uniform64(__shfl(cc.incl, 63));
      if (cs < base + total) {
        pick(cc);
        break;
      }
      base += total;
    }
  }
  if (s_found < 0) {
    zero_rows();
    return;
  }
  load_chunk(s0);

  auto len_of = [&](int s) -> int {  // decode length of sequence s (chunk reloaded on demand)
    if (s >= s0 + 256) {
      s0 = s - (s - s0) % 256;
      wave_sync();
      load_chunk(s0);
    }
    return uniform(len_lds[s - s0]);
  };
  auto row_of = [&](int s) -> int { return uniform(row_lds[s - s0]); };

  StreamCur cur0;
  {
    const int L = len_of(s_found);
    const int n = (L + SS::STEP - 1) / SS::STEP;
    const long long h = (cs - S_found) / (n + c0);
    cur0.s = s_found;
    cur0.h = (int)h;
    cur0.n = n;
    cur0.L = L;
    cur0.row = row_of(s_found);
    cur0.A = S_found + h * (n + c0) + c0;
    cur0.j = (int)max(0LL, cs - cur0.A);
    cur0.valid = cur0.A + cur0.j < ce;
  }
  if (!cur0.valid) {
    zero_rows();
    return;
  }

  auto next = [&](const StreamCur& c) {
    StreamCur r = c;
    if (!c.valid) return r;
    if (c.j + 1 < c.n) {
      r.j = c.j + 1;
      r.valid = c.A + r.j < ce;
      return r;
    }
    r.A = c.A + c.n + c0;
    r.j = 0;
    if (r.A >= ce) {
      r.valid = 0;
      return r;
    }
    if (c.h + 1 < hkv) {
      r.h = c.h + 1;
      return r;
    }
    int s = c.s + 1;
    int L = 0;
    while (s < p.num_seqs && (L = len_of(s)) <= 0) ++s;
    if (s >= p.num_seqs) {
      r.valid = 0;
      return r;
    }
    r.s = s;
    r.h = 0;
    r.L = L;
    r.n = (L + SS::STEP - 1) / SS::STEP;
    r.row = row_of(s);
    return r;
  };

  // block ids of a step: lane l gets block NB j + k of the item's row, k =
  // l / 16 (four-block steps: the block of the lane's token) or l % NB;
  // lane id_lane(k) holds block k.
  auto id_lane = [](int k) { return SS::TPL ? 16 * k : k; };
  auto load_ids = [&](const StreamCur& c) -> int {
    const int nblk = (c.L + BS - 1) / BS;
    const int b = min(SS::NB * c.j + (SS::TPL ? lane >> 4 : lane % SS::NB), nblk - 1);
    return p.block_tables[(size_t)c.s * p.max_blocks + b];
  };
  auto load_q = [&](uint4 (&qr)[NQ], const StreamCur& c) {
    const uint4* src = reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) + ((size_t)c.row * hq + (size_t)c.h * G) * D * S::QES);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int gi = lane + 64 * i;
      qr[i] = (gi < QGR) ? src[gi] : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_q = [&](const uint4 (&qr)[NQ]) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int gi = lane + 64 * i;
      if (gi < QGR) {
        const int g = gi / S::QKG, c = gi % S::QKG;
        const int hh = c / S::QKH, cc = c % S::QKH;
        *reinterpret_cast<uint4*>(q_lds + (g * 2 + hh) * S::QROW + cc * 16) = qr[i];
      }
    }
  };

  const int half = lane & 1;
  const int t_in_blk = (lane >> 1) & 15;
  const int bsel = lane >> 5;
  const int k_lane_off = (half * S::KH * BS + t_in_blk) * 16;
  // K/V of a step whose blocks are lb[0 .. NB) (lid: the lane's value of
  // the same ids): the lane's K granules (four-block steps: token lane of
  // the step, in block lane / 16, the whole row; otherwise token t_in_blk of
  // block bsel, half row `half`), then the V tiles, one granule per d and
  // block.
  auto load_kv = [&](StreamRegs<ES, D, G>& r, int h, const int (&lb)[SS::NB], int lid) {
    const char* head_base = p.kv + (size_t)h * 2 * S::TILE;
    const char* kp;
    if constexpr (SS::TPL) {
      kp = head_base + (size_t)lid * p.block_bytes + (lane & 15) * 16;
    } else {
      kp = head_base + (size_t)(bsel ? lb[1] : lb[0]) * p.block_bytes + k_lane_off;
    }
#pragma unroll
    for (int cc = 0; cc < SS::KL; ++cc) r.k[cc] = load_once(kp + cc * BS * 16);
#pragma unroll
    for (int i = 0; i < S::VG; ++i)
#pragma unroll
      for (int jb = 0; jb < SS::NB; ++jb)
        r.v[jb][i] = load_once(head_base + (size_t)lb[jb] * p.block_bytes + S::TILE + i * 1024 +
                               lane * 16);
  };

  float m_run[G], l_lane[G], acc[G][S::DPL];
  auto reset_state = [&]() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.f;
#pragma unroll
      for (int j = 0; j < S::DPL; ++j) acc[g][j] = 0.f;
    }
  };

  auto compute = [&](const StreamRegs<ES, D, G>& r, const StreamCur& c) {
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    const char* qh = q_lds + half * S::QROW;
    if constexpr (ES == 1) {
      // The lane's token against every head: K granule cc holds the 16 E4M3
      // codes of d = 16 cc .., converted pairwise to bf16 (exact) for v_dot2
      // against q granules 2 cc and 2 cc + 1 (one half row holds both).
#pragma unroll
      for (int cc = 0; cc < SS::KL; ++cc) {
        const uint4 kg = r.k[cc];
        const uint32_t kw[4] = {kg.x, kg.y, kg.z, kg.w};
        uint32_t kb[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          kb[2 * q] = fp8x2_bf16<false>(kw[q]);
          kb[2 * q + 1] = fp8x2_bf16<true>(kw[q]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const char* qp = q_lds + (g * 2 + 2 * cc / S::QKH) * S::QROW + (2 * cc % S::QKH) * 16;
          const uint4 q0 = *reinterpret_cast<const uint4*>(qp);
          const uint4 q1 = *reinterpret_cast<const uint4*>(qp + 16);
          const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[e]),
                                                    __builtin_bit_cast(bf16x2_t, kb[e]), sc[g], false);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) asm volatile("" : "+v"(sc[g]));
      }
    } else if constexpr (SS::TPL) {
      // bf16, the lane's token against every head: K granule cc and q
      // granule cc hold the same 8 d values
#pragma unroll
      for (int cc = 0; cc < SS::KL; ++cc) {
        const uint4 kg = r.k[cc];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint4 qg = *reinterpret_cast<const uint4*>(
              q_lds + (g * 2 + cc / S::QKH) * S::QROW + (cc % S::QKH) * 16);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.x),
                                                  __builtin_bit_cast(bf16x2_t, kg.x), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.y),
                                                  __builtin_bit_cast(bf16x2_t, kg.y), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.z),
                                                  __builtin_bit_cast(bf16x2_t, kg.z), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.w),
                                                  __builtin_bit_cast(bf16x2_t, kg.w), sc[g], false);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) asm volatile("" : "+v"(sc[g]));
      }
    } else {
    uint4 qcur[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qcur[g] = *reinterpret_cast<const uint4*>(qh + g * 2 * S::QROW);
#pragma unroll
    for (int cc = 0; cc < S::KH; ++cc) {
      uint4 qnext[G];
      const int cn = cc + 1 < S::KH ? cc + 1 : cc;
#pragma unroll
      for (int g = 0; g < G; ++g)
        qnext[g] = *reinterpret_cast<const uint4*>(qh + g * 2 * S::QROW + cn * 16);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 qg = qcur[g];
        const uint4 kg = r.k[cc];
        if constexpr (ES == 2) {
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.x),
                                                  __builtin_bit_cast(bf16x2_t, kg.x), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.y),
                                                  __builtin_bit_cast(bf16x2_t, kg.y), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.z),
                                                  __builtin_bit_cast(bf16x2_t, kg.z), sc[g], false);
          sc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qg.w),
                                                  __builtin_bit_cast(bf16x2_t, kg.w), sc[g], false);
        } else {
          sc[g] = fmaf(__uint_as_float(qg.x), __uint_as_float(kg.x), sc[g]);
          sc[g] = fmaf(__uint_as_float(qg.y), __uint_as_float(kg.y), sc[g]);
          sc[g] = fmaf(__uint_as_float(qg.z), __uint_as_float(kg.z), sc[g]);
          sc[g] = fmaf(__uint_as_float(qg.w), __uint_as_float(kg.w), sc[g]);
        }
        qcur[g] = qnext[g];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) asm volatile("" : "+v"(sc[g]));
    }
    }
    const int tok0 = c.j * SS::STEP;
    const bool tok_ok = tok0 + (SS::TPL ? lane : lane >> 1) < c.L;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float full = SS::TPL ? sc[g] : sc[g] + dpp_f<0xB1>(sc[g]);
      const float x = tok_ok ? full * p.scale_log2 : -INFINITY;
      const float mi = wave_max(x);
      if (mi > m_run[g] + kRescaleSlack) {
        const float corr = __builtin_amdgcn_exp2f(m_run[g] - mi);
        l_lane[g] *= corr;
#pragma unroll
        for (int j = 0; j < S::DPL; ++j) acc[g][j] *= corr;
        m_run[g] = mi;
      }
      const float pr = __builtin_amdgcn_exp2f(x - m_run[g]);
      if constexpr (ES == 1) {  // fp16 probabilities; the sums use the same rounded values
        const _Float16 ph = (_Float16)pr;
        l_lane[g] += (float)ph;
        reinterpret_cast<_Float16*>(p_lds)[g * SS::STEP + lane] = ph;
      } else if (SS::TPL) {
        l_lane[g] += pr;
        p_lds[lane * G + g] = pr;
      } else if (half == 0) {
        l_lane[g] += pr;
        p_lds[(lane >> 1) * G + g] = pr;
      }
    }
    wave_sync();
#pragma unroll
    for (int jb = 0; jb < SS::NB; ++jb) {
      const int valid = c.L - (tok0 + jb * BS);
      if constexpr (ES == 1) {
        const uint16_t* p16 = reinterpret_cast<const uint16_t*>(p_lds);
        if (valid >= BS)
          pv_block_fp8<D, G, false, SS::STEP>(r.v[jb], p16, jb * BS, BS, acc);
        else if (valid > 0)
          pv_block_fp8<D, G, true, SS::STEP>(r.v[jb], p16, jb * BS, valid, acc);
      } else {
        if (valid >= BS)
          pv_block<ES, D, G, false>(r.v[jb], p_lds, jb * BS, BS, acc);
        else if (valid > 0)
          pv_block<ES, D, G, true>(r.v[jb], p_lds, jb * BS, valid, acc);
      }
    }
    wave_sync();
  };

  // Split items this wave has left a partial for.
  struct Pending {
    int ctr, wA, wB, row, h;
  };
  Pending pend0 = {0, 0, 0, 0, 0}, pend1 = {0, 0, 0, 0, 0};
  int npend = 0;

  // The item of `c` ends here (its last step in this wave's range).
  auto finish = [&](const StreamCur& c) {
    float l_tot[G];
#pragma unroll
    for (int g = 0; g < G; ++g) l_tot[g] = wave_sum(l_lane[g]);
    const int wA = stream_wave_of(split, c.A, T);
    const int wB = stream_wave_of(split, c.A + c.n - 1, T);
    float* o = p.out + ((size_t)c.row * hq + (size_t)c.h * G) * D;
    if (wA == wB) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < S::DPL; ++j)
          o[g * D + j * 64 + lane] = acc[g][j] / l_tot[g] * p.out_scale;
      reset_state();
      return;
    }
    const int slot = 2 * w + (w == wA ? 1 : 0);
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < S::DPL; ++j)
        store_agent(sp.part_acc + ((size_t)slot * G + g) * D + j * 64 + lane, acc[g][j]);
      if (lane == 0) {
        store_agent(sp.part_ml + ((size_t)slot * G + g) * 2, m_run[g]);
        store_agent(sp.part_ml + ((size_t)slot * G + g) * 2 + 1, l_tot[g]);
      }
    }
    reset_state();
    // counted and merged after the walk (at most two split items per wave:
    // the first and the last of its range)
    if (npend == 0) {
      pend0 = {c.s * hkv + c.h, wA, wB, c.row, c.h};
    } else {
      pend1 = {c.s * hkv + c.h, wA, wB, c.row, c.h};
    }
    ++npend;
  };

  // ---- the walk.  Two register sets alternate: ra holds the step being
  // computed while rb receives the next one, then the roles swap.  Every
  // step issues the same loads (the next step's K/V, the block ids of the
  // step two after), so the compiler's wait counts stay exact on all paths:
  // past the end of the range the ids come from the current step and the
  // K/V are a re-read of the current step's blocks (an L2 hit).  Ids
  // loaded two steps ahead have arrived when their K/V are issued; loaded
  // one step ahead, the issue could wait on a load only one step old (8B
  // GQA batch: 0.674-0.676 of 8 TB/s against 0.669-0.671).
  StreamRegs<ES, D, G> ra, rb;
  uint4 qa[NQ], qb[NQ];
  load_q(qa, cur0);
  int ids_a = load_ids(cur0);  // ids of the step whose K/V go to ra
  StreamCur cur1 = next(cur0);
  int ids_1 = load_ids(cur1.valid ? cur1 : cur0);
  StreamCur cur2 = next(cur1);
  int ids_2 = load_ids(cur2.valid ? cur2 : cur0);
  int lb[SS::NB];  // blocks of the last K/V issued
  int lid = 0;     // the same, as load_ids gave them to this lane
  auto take_ids = [&](int ids) {
#pragma unroll
    for (int k = 0; k < SS::NB; ++k) lb[k] = uniform(__builtin_amdgcn_readlane(ids, id_lane(k)));
    lid = ids;
  };
  take_ids(ids_a);
  load_kv(ra, cur0.h, lb, lid);
  bool new0 = true;
  reset_state();

  // One step: compute `c` (data in rc, q rows in qc if it starts an item),
  // with `cn` = the step after (K/V -> rn, q -> qn; its ids in ids_n) and
  // `cf` the one after that (ids in ids_f); loads the ids of the step after
  // `cf`, which it returns, and shifts ids_f into ids_n.
  auto half_step = [&](StreamRegs<ES, D, G>& rc, StreamRegs<ES, D, G>& rn, uint4 (&qc)[NQ], uint4 (&qn)[NQ],
                       const StreamCur& c, StreamCur& cn, const StreamCur& cf, int& ids_n, int& ids_f,
                       bool& new_c) {
    StreamCur c2 = next(cf);
    const bool new_n = cn.valid && (cn.s != c.s || cn.h != c.h);
    if (new_n) load_q(qn, cn);
    const int ids_new = load_ids(c2.valid ? c2 : c);
    int hh = c.h;
    if (cn.valid) {
      take_ids(ids_n);
      hh = cn.h;
    }
    ids_n = ids_f;
    ids_f = ids_new;
    load_kv(rn, hh, lb, lid);
    if (new_c) {
      store_q(qc);
      wave_sync();
    }
    compute(rc, c);
    if (!cn.valid || new_n) finish(c);
    new_c = new_n;
    return c2;
  };

  // sp.rounds waves share each SIMD (waves w, w + W / rounds, ... in
  // dispatch order), and the issue arbiter favours the oldest: with equal
  // work, the second of two waves ended ~40 us after the first.  Each wave
  // steps its priority through 0 .. rounds - 1, one step per step of the
  // walk, starting at its dispatch round, so the waves of a SIMD take turns
  // at the top and advance at about the same rate.  (Beside prefill tiles,
  // one decode wave per SIMD, rounds is 0: off.)
  const int rounds = sp.rounds;
  int ph = uniform(rounds > 1 ? (int)((long long)w * rounds / W) : 0);
  auto next_priority = [&]() {
    if (rounds > 1) {
      if (ph == 0) __builtin_amdgcn_s_setprio(0);
      else if (ph == 1) __builtin_amdgcn_s_setprio(1);
      else if (ph == 2) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(3);
      ph = ph + 1 == rounds ? 0 : ph + 1;
    }
  };
  for (;;) {
    next_priority();
    StreamCur c3 = half_step(ra, rb, qa, qb, cur0, cur1, cur2, ids_1, ids_2, new0);
    if (!cur1.valid) break;
    cur0 = cur1;
    cur1 = cur2;
    cur2 = c3;
    next_priority();
    StreamCur c4 = half_step(rb, ra, qb, qa, cur0, cur1, cur2, ids_1, ids_2, new0);
    if (!cur1.valid) break;
    cur0 = cur1;
    cur1 = cur2;
    cur2 = c4;
  }

  zero_rows();
  // ---- count this wave into its split items (lanes 0 and 1 at once, after
  // its partial stores are complete); the last contributor merges.
  if (npend == 0) return;
  wait_stores();
  unsigned cnt = 0;
  if (lane < npend) {
    unsigned long long* ctr = sp.counters + (lane == 0 ? pend0.ctr : pend1.ctr);
    const unsigned long long tag = (unsigned long long)sp.epoch << 32;
    unsigned long long seen = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
      const unsigned long long want = ((seen >> 32) == sp.epoch) ? seen + 1 : (tag | 1ULL);
      const unsigned long long prev = atomicCAS(ctr, seen, want);
      if (prev == seen) {
        cnt = (unsigned)want;
        break;
      }
      seen = prev;
    }
  }
  const unsigned cnt0 = (unsigned)__builtin_amdgcn_readlane((int)cnt, 0);
  const unsigned cnt1 = (unsigned)__builtin_amdgcn_readlane((int)cnt, 1);
  const bool last0 = cnt0 == (unsigned)(pend0.wB - pend0.wA + 1);
  const bool last1 = npend > 1 && cnt1 == (unsigned)(pend1.wB - pend1.wA + 1);
  // Every contributor has counted itself in: no wave of this call touches
  // these counters again.
  if ((lane == 0 && last0) || (lane == 1 && last1))
    __hip_atomic_store(sp.counters + (lane == 0 ? pend0.ctr : pend1.ctr), 0ULL, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (last0)
    stream_merge<ES, D, G>(sp, pend0.wA, pend0.wB,
                           p.out + ((size_t)pend0.row * hq + (size_t)pend0.h * G) * D);
  if (last1)
    stream_merge<ES, D, G>(sp, pend1.wA, pend1.wB,
                           p.out + ((size_t)pend1.row * hq + (size_t)pend1.h * G) * D);
}

template <int ES, int D, int G>
static hipError_t decode_rows_t(const DecodeParams& p, int64_t units, int num_seqs, int hkv,
                                hipStream_t stream) {
  if (units > 0) {
    const int64_t items = units * hkv;
    hipLaunchKernelGGL((k_decode_partition<ES, D, G>), dim3((unsigned)items), dim3(64), 0, stream,
                       p);
  }
  if (num_seqs > 0)
    hipLaunchKernelGGL((k_decode_merge<D, G>), dim3((unsigned)((int64_t)num_seqs * hkv)),
                       dim3(64 * (G < 4 ? G : 4)), 0, stream, p);
  return hipGetLastError();
}

template <int ES, int D>
static hipError_t decode_rows_g(int G, const DecodeParams& p, int64_t units, int num_seqs, int hkv,
                                hipStream_t stream) {
  switch (G) {
    case 1: return decode_rows_t<ES, D, 1>(p, units, num_seqs, hkv, stream);
    case 2: return decode_rows_t<ES, D, 2>(p, units, num_seqs, hkv, stream);
    case 4: return decode_rows_t<ES, D, 4>(p, units, num_seqs, hkv, stream);
    case 8: return decode_rows_t<ES, D, 8>(p, units, num_seqs, hkv, stream);
  }
  return hipErrorInvalidValue;
}

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

static DecodeParams make_decode_params(const CacheDesc& c, const AttnDesc& a) {
  DecodeParams p;
  p.kv = c.kv;
  p.block_bytes = c.block_bytes;
  p.hkv = c.hkv;
  p.q = a.q;
  p.out = a.out;
  p.block_tables = a.block_tables;
  p.max_blocks = a.max_blocks;
  p.seq_lens = a.seq_lens;
  p.qsl = a.query_start_loc;
  p.num_seqs = a.num_seqs;
  p.scale_log2 = a.scale * kLog2e;
  p.out_scale = a.out_scale;
  p.ws_acc = a.ws_acc;
  p.ws_ml = a.ws_ml;
  p.full_units = (int)a.full_units;
  p.total_items = (int)(a.decode_units * c.hkv);
  for (int k = 0; k <= kPartClasses; ++k) p.class_start[k] = (int)a.class_start[k];
  return p;
}

template <int ES, int D, int G>
static hipError_t stream_t(const StreamParams& sp, hipStream_t stream) {
  hipLaunchKernelGGL((k_decode_stream<ES, D, G>), dim3((unsigned)sp.waves), dim3(64), 0, stream, sp);
  return hipGetLastError();
}

template <int ES, int D>
static hipError_t stream_g(int G, const StreamParams& sp, hipStream_t stream) {
  switch (G) {
    case 1: return stream_t<ES, D, 1>(sp, stream);
    case 2: return stream_t<ES, D, 2>(sp, stream);
    case 4: return stream_t<ES, D, 4>(sp, stream);
    case 8: return stream_t<ES, D, 8>(sp, stream);
  }
  return hipErrorInvalidValue;
}

template <int ES, int D, int G>
static int stream_blocks_per_cu() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_stream<ES, D, G>, 64, 0) !=
      hipSuccess)
    return 0;
  return nb;
}

int decode_stream_slots(int dtype_bytes, int D, int G) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int nb = 0;
#define PKV_SLOTS(ES_, D_)                                 \
  switch (G) {                                             \
    case 1: nb = stream_blocks_per_cu<ES_, D_, 1>(); break; \
    case 2: nb = stream_blocks_per_cu<ES_, D_, 2>(); break; \
    case 4: nb = stream_blocks_per_cu<ES_, D_, 4>(); break; \
    case 8: nb = stream_blocks_per_cu<ES_, D_, 8>(); break; \
  }
  if (dtype_bytes == 1 && D == 64) { PKV_SLOTS(1, 64) }
  else if (dtype_bytes == 1 && D == 128) { PKV_SLOTS(1, 128) }
  else if (dtype_bytes == 4 && D == 64) { PKV_SLOTS(4, 64) }
  else if (dtype_bytes == 4 && D == 128) { PKV_SLOTS(4, 128) }
  else if (dtype_bytes == 2 && D == 64) { PKV_SLOTS(2, 64) }
  else if (dtype_bytes == 2 && D == 128) { PKV_SLOTS(2, 128) }
#undef PKV_SLOTS
  // Measured on MI355X (8B GQA batch 256, 1 GiB of other data read before
  // every call so that neither the Infinity Cache nor the TLBs hold the last
  // call's blocks):
  //  - bf16: two waves per SIMD, 0.267 ms against 0.284 ms with one, whose
  //    single chain of requests hides those misses less well (back to back,
  //    with the blocks still cached, one wave is the faster: 0.260 vs 0.267);
  //  - fp8: two waves per SIMD of four-block steps (two-block steps, the
  //    earlier design, wanted three waves and still streamed slower);
  //  - bf16 with one query head per kv head at D = 128: one wave per SIMD
  //    of four-block steps (its registers need the whole file).
  const int per_cu = 8;
  return (nb < per_cu ? nb : per_cu) * cus;
}

static hipError_t launch_decode_stream(const CacheDesc& c, const AttnDesc& a, hipStream_t stream) {
  StreamParams sp;
  sp.d = make_decode_params(c, a);
  sp.waves = a.stream_waves;
  sp.c0 = a.stream_c0;
  sp.epoch = a.stream_epoch;
  sp.rounds = a.stream_rounds;
  for (int k = 0; k < 4; ++k) sp.wt[k] = a.stream_wt[k];
  sp.half = a.stream_half;
  sp.counters = a.stream_counters;
  sp.part_acc = a.stream_acc;
  sp.part_ml = a.stream_ml;
  const int G = a.hq / c.hkv;
  if (c.dtype_bytes == 1) {
    if (c.head_size == 64) return stream_g<1, 64>(G, sp, stream);
    if (c.head_size == 128) return stream_g<1, 128>(G, sp, stream);
  } else if (c.dtype_bytes == 4) {
    if (c.head_size == 64) return stream_g<4, 64>(G, sp, stream);
    if (c.head_size == 128) return stream_g<4, 128>(G, sp, stream);
  } else {
    if (c.head_size == 64) return stream_g<2, 64>(G, sp, stream);
    if (c.head_size == 128) return stream_g<2, 128>(G, sp, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_rows(const CacheDesc& c, const AttnDesc& a, hipStream_t stream) {
  const DecodeParams p = make_decode_params(c, a);
  if (a.stream_waves > 0) return launch_decode_stream(c, a, stream);
  if (c.fp8) return hipErrorInvalidValue;  // fp8 caches are read by the stream kernel only
  const int G = a.hq / c.hkv;
  if (c.dtype_bytes == 4) {
    if (c.head_size == 64) return decode_rows_g<4, 64>(G, p, a.decode_units, a.num_seqs, c.hkv, stream);
    if (c.head_size == 128) return decode_rows_g<4, 128>(G, p, a.decode_units, a.num_seqs, c.hkv, stream);
  } else {
    if (c.head_size == 64) return decode_rows_g<2, 64>(G, p, a.decode_units, a.num_seqs, c.hkv, stream);
    if (c.head_size == 128) return decode_rows_g<2, 128>(G, p, a.decode_units, a.num_seqs, c.hkv, stream);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Prefill rows of a mixed batch (chunked prefill, juhe.plus section 4.2):
// sequence s has q_len > 1 query rows at positions L - q_len .. L - 1, each
// seeing keys 0..its position.  Both products are dense here, so they run
// on MFMA:
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16 (32 keys x 32 query rows, k = d)
//   O^T += V^T P^T v_mfma_f32_32x32x16_f16  (32 d x 32 query rows, k = keys)
// Computing S transposed leaves each lane with one query row, so the
// softmax row max needs a single exchange between the two 32-lane halves,
// and the S^T accumulator is already the B operand of the second product.
//
// Precision of P.V: probabilities and V enter the second product as fp16
// (11 significant bits; bf16's 8 would leave a relative error near 1e-3).
// A first pass (k_v_fp16) converts the V tiles of every prefill sequence's
// blocks once, through the block table, into the workspace: each block
// tile is scaled by the power of two 2^-e (exact) that keeps it below 2^16,
// e is recorded per (kv head, block), and keys past the sequence length are
// zeroed.  The tile kernel keeps its accumulator in units of 2^kexp and
// adjusts P or the accumulator by exact powers of two when a block's e
// differs (all e are 0 unless some |v| >= 2^16).  The row sums l come from
// the same rounded fp16 probabilities that enter the MFMA (v_fma_mix_f32,
// before any such adjustment), so the normalisation matches the weights.
//
// One workgroup = 4 waves = one kv head x TQ positions; wave w takes query
// head w % G of the group and positions 32*(w / G) .. +31 of the tile.
// Keys arrive 64 at a time (4 blocks): wave w copies block w's K tile
// (from the pool, through the block table) and fp16 V tile (from the
// workspace) straight into LDS with global_load_lds_dwordx4, in their HBM
// layouts, two stages deep, so one barrier per tile suffices and no
// registers stage the data.  The K operand's lane r reads key pi(r), where
// pi swaps bits 2 and 3 of r: the S^T rows a lane then holds are the 8
// consecutive keys of one V granule, which is the k order of the second
// product's operands, so both operand fragments are single 16-byte reads.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

struct PrefillParams {
  const char* kv;
  size_t block_bytes;
  int hkv;
  const uint16_t* q;
  float* out;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int num_seqs;
  float scale_log2;
  char* vh;          // fp16 V tiles [vblock][hkv][16 * D], vblock = sequence-major
  int32_t* vexp;     // scale exponents [hkv][vblocks]
  int64_t vblocks;   // blocks of all prefill sequences, each rounded up to 4
  int items;         // prefill q tiles over all sequences (workgroups / hkv)
  int pair_from;     // > 0: item slots >= pair_from run the lightest items in reverse
  int prio;          // 1: the tile waves raise their issue priority (beside decode waves)
};

template <int D, int G>
struct PrefillShape {
  static constexpr int TQ = prefill_tile_q(G);  // query positions per workgroup
  static constexpr int KT = 64;                 // keys per tile (4 blocks)
  static constexpr int KS = D / 16;             // MFMA k-steps over the head dim
  static constexpr int DB = D / 32;             // 32-row d blocks of O^T
  static constexpr int TILE = BS * D * 2;       // bytes of one block's K (or fp16 V) tile
  static constexpr int BUF = 4 * TILE;          // one tile's K (or V): 4 blocks
  static constexpr int CP = TILE / 1024;        // 1 KiB copies per tile and wave
};


// Find (sequence, item, items of that sequence) of work item u, where
// count(s) gives the items of sequence s.  Every lane gets the result.
template <typename F>
__device__ bool find_item(int u, int num_seqs, F count, int& s_out, int& item_out, int& n_out) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int s0 = 0; s0 < num_seqs; s0 += 64) {
    const int s = s0 + lane;
    const int n = (s < num_seqs) ? count(s) : 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int total = __shfl(incl, 63);
    if (u < base + total) {
      const unsigned long long m = __ballot(base + incl > u);
      const int ls = __ffsll((unsigned long long)m) - 1;
      const int incl_s = __shfl(incl, ls);
      const int n_s = __shfl(n, ls);
      s_out = uniform(s0 + ls);
      item_out = uniform(u - (base + incl_s - n_s));
      n_out = uniform(n_s);
      return true;
    }
    base += total;
  }
  return false;
}

// Sum of count(q) over sequences q < s (wave-level; every lane gets it).
template <typename F>
__device__ int count_before(int s, F count) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int s0 = 0; s0 < s; s0 += 64) {
    int v = (s0 + lane < s) ? count(s0 + lane) : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    sum += v;
  }
  return uniform(sum);
}

// Blocks of prefill sequence q converted by k_v_fp16 (0 for decode rows).
__device__ __forceinline__ int prefill_vblocks_of(const PrefillParams& p, int q) {
  const int ql = p.qsl[q + 1] - p.qsl[q];
  return ql > 1 ? 4 * ((p.seq_lens[q] + 4 * BS - 1) / (4 * BS)) : 0;
}

// Max of the two 32-lane halves of the wave, in every lane.
__device__ __forceinline__ float half_swap_max(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                   false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float half_swap_sum(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                   false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Two fp32 -> two fp16 (round to nearest even) packed in one dword.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float bf16x2_absmax(uint32_t w) {
  return fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w)));
}

// ---- V tiles of the prefill sequences -> fp16 in the workspace.  One wave
// per (vblock, kv head): the tile's 16 * D values, keys >= L zeroed, scaled
// by 2^-e with e the smallest exponent that brings every |v| below 2^16.
template <int D>
__global__ __launch_bounds__(256) void k_v_fp16(PrefillParams p) {
  if (p.prio) __builtin_amdgcn_s_setprio(3);
  constexpr int TILE = BS * D * 2;
  constexpr int NG = TILE / 16 / 64;  // granules per lane
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.vblocks * p.hkv) return;
  const int kvh = (int)(item % p.hkv);
  const int vb = (int)(item / p.hkv);
  int s, j, n;
  if (!find_item(vb, p.num_seqs, [&p](int q) { return prefill_vblocks_of(p, q); }, s, j, n)) return;
  const int L = uniform(p.seq_lens[s]);
  uint4 g[NG];
  if (j * BS < L) {
    const int id = uniform(p.block_tables[(size_t)s * p.max_blocks + j]);
    const char* src = p.kv + (size_t)id * p.block_bytes + (size_t)(2 * kvh + 1) * TILE;
#pragma unroll
    for (int i = 0; i < NG; ++i) g[i] = load_once(src + (lane + 64 * i) * 16);
    if (j * BS + BS > L) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int key0 = j * BS + ((lane + 64 * i) / D) * 8;  // granule = 8 keys of one d
        uint32_t w[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (key0 + e >= L) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        g[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NG; ++i) g[i] = make_uint4(0, 0, 0, 0);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < NG; ++i)
    m = fmaxf(m, fmaxf(fmaxf(bf16x2_absmax(g[i].x), bf16x2_absmax(g[i].y)),
                       fmaxf(bf16x2_absmax(g[i].z), bf16x2_absmax(g[i].w))));
  m = wave_max(m);
  // smallest e >= 0 with m * 2^-e < 2^16; non-finite maxima get a bounded e
  // (their results are then non-finite as in exact arithmetic)
  const int ex = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;
  const int e = min(max(ex - 15, 0), 100);
  const float sc = __builtin_ldexpf(1.f, -e);
  char* dst = p.vh + ((size_t)vb * p.hkv + kvh) * TILE;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const uint4 v = g[i];
    *reinterpret_cast<uint4*>(dst + (lane + 64 * i) * 16) = make_uint4(
        pack_f16x2(bf16_lo(v.x) * sc, bf16_hi(v.x) * sc), pack_f16x2(bf16_lo(v.y) * sc, bf16_hi(v.y) * sc),
        pack_f16x2(bf16_lo(v.z) * sc, bf16_hi(v.z) * sc), pack_f16x2(bf16_lo(v.w) * sc, bf16_hi(v.w) * sc));
  }
  if (lane == 0) p.vexp[(size_t)kvh * p.vblocks + vb] = e;
}

// One prefill work item (q tile, kv head) on a whole 4-wave workgroup.
// `kb0`, `kb1` (K) and `vb0`, `vb1` (V) are double buffers of one 64-key
// tile each (4 blocks).  They must be distinct __shared__ arrays: the
// compiler then sees that the copies into one buffer cannot alias the reads
// of another and does not make the reads wait for those copies.
// VB: V is read as bf16 straight from the pool (through the block table,
// like K) and P enters the P.V product as a bf16 hi + lo pair (two MFMAs);
// otherwise V comes from the fp16 copy k_v_fp16 made in the workspace.
// SPLIT: the workgroup has 8 waves in two groups of 4 that hold the same
// query rows; group `grp` takes one half of the item's key tiles (group 0
// the first ceil(n / 2), group 1 the rest) into its own buffers, and at the
// end group 1 hands its (max, sum, O) to group 0 through LDS (`xo0`, `xo1`:
// two waves' O each; `xml`: max, sum and exponent), which merges and writes
// the rows.  Both groups run the same number of tile iterations, so they
// meet at every barrier.
template <int D, int G, bool VB, bool SPLIT = false>
__device__ __forceinline__ void prefill_item(const PrefillParams& p, int work, char* kb0,
                                             char* kb1, char* vb0, char* vb1, int grp = 0,
                                             char* xo0 = nullptr, char* xo1 = nullptr,
                                             char* xml = nullptr) {
  static_assert(!(SPLIT && VB), "the split runs the fp16-V path only");
  using S = PrefillShape<D, G>;
  static_assert(G == 1 || G == 2 || G == 4, "4 waves cover at most 4 query heads");
  constexpr int KS = S::KS, DB = S::DB;
  constexpr int PVN = (VB ? 4 : 2) * DB;  // P.V products per 32-key chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform((tid >> 6) & 3);
  const int kvh = work % p.hkv;
  int item = work / p.hkv;
  // The dispatcher gives workgroup w + (CU count) the CU of workgroup w.  With
  // at most two workgroups per CU, the first round takes the heaviest items
  // (latest q tiles first) and the second round the rest from the lightest
  // up, so the two items that share a CU add up to about the same key range
  // on every CU.  The kv head stays work % hkv (one head's K/V per XCD's L2).
  if (p.pair_from > 0 && item >= p.pair_from) item = p.items - 1 + p.pair_from - item;
  int s, tile, ntiles;
  const int32_t* qsl = p.qsl;
  auto tiles_of = [qsl](int q) __attribute__((always_inline)) {
    const int ql = qsl[q + 1] - qsl[q];
    return ql > 1 ? (ql + S::TQ - 1) / S::TQ : 0;
  };
  if (!find_item(item, p.num_seqs, tiles_of, s, tile, ntiles)) return;
  tile = ntiles - 1 - tile;  // later tiles see more keys: dispatch them first
  const int vbase = count_before(s, [&p](int q) { return prefill_vblocks_of(p, q); });

  const int hq = p.hkv * G;
  const int L = uniform(p.seq_lens[s]);
  const int row0 = uniform(qsl[s]);
  const int ql = uniform(qsl[s + 1]) - row0;
  const int qfirst = L - ql;                       // position of query row 0
  const int p0 = qfirst + tile * S::TQ;
  const int pend = min(qfirst + ql, p0 + S::TQ);   // positions [p0, pend)
  const int g = wave % G;
  const int wp0 = p0 + 32 * (wave / G);
  const int wlast = min(wp0 + 31, pend - 1);       // < wp0 when the wave has no rows
  const int h = lane >> 5;
  const int r = lane & 31;
  const int my_pos = wp0 + r;
  const bool row_ok = my_pos < pend;
  const int lim = row_ok ? my_pos : -1;            // last key this row sees
  const int head = kvh * G + g;

  // A negative scale is carried by negating q (exact), so that c > 0 and
  // the largest raw score is the largest scaled one; a zero scale becomes
  // the least normal float, so masked scores (-inf) still give exp2 = 0.
  const bool neg = p.scale_log2 < 0.f;
  const float c = fmaxf(fabsf(p.scale_log2), 1.17549435e-38f);

  // Q^T operand: lane (h, r) holds q[row r][16 ks + 8 h .. + 8] for every ks.
  bf16x8_t qb[S::KS];
  {
    const size_t tok = (size_t)row0 + (size_t)(row_ok ? my_pos - qfirst : 0);
    const uint4* qrow = reinterpret_cast<const uint4*>(p.q + (tok * hq + head) * D);
    const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      uint4 v = row_ok ? qrow[2 * ks + h] : make_uint4(0, 0, 0, 0);
      v.x ^= flip; v.y ^= flip; v.z ^= flip; v.w ^= flip;
      qb[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  const int nkt = uniform((pend + S::KT - 1) / S::KT);  // key tiles needed (keys < pend)
  const int nbl = uniform((L + BS - 1) / BS);           // valid block-table entries
  // 32-key chunks this wave needs (keys up to its last row's position)
  const int nch = uniform(wlast >= wp0 ? wlast / 32 + 1 : 0);
  // This group's key tiles [tb, te) and chunks [c_beg, c_end); niter tile
  // iterations (the same in both groups of a split workgroup).
  const int half_t = (nkt + 1) / 2;
  const int tb = SPLIT && grp ? half_t : 0;
  const int te = SPLIT && !grp ? half_t : nkt;
  const int niter = SPLIT ? half_t : nkt;
  const int c_beg = 2 * tb;
  const int c_end = uniform(min(nch, 2 * te));
  const char* k_src = p.kv + (size_t)kvh * 2 * S::TILE + lane * 16;
  const char* v_src = VB ? p.kv + (size_t)(2 * kvh + 1) * S::TILE + lane * 16
                        : p.vh + ((size_t)vbase * p.hkv + kvh) * S::TILE + lane * 16;

  // Per-tile metadata travels in one vector load issued with the copies of
  // the iteration before (scalar loads would make every later LDS wait also
  // wait for them).  Iteration t reads lanes 0..3: block ids of tile t + 2
  // (its K copies start in iteration t); lanes 4..7: VB, the ids of tile
  // t + 1 (its V copies start in iteration t), else the V exponents of tile t.
  const int32_t* bt_row = p.block_tables + (size_t)s * p.max_blocks;
  const int32_t* exp_row = p.vexp + (size_t)kvh * p.vblocks + vbase;
  int meta = bt_row[min(4 * tb + (lane & 7), nbl - 1)];  // before the loop: ids of tiles tb, tb + 1
  auto load_meta = [&](int t) __attribute__((always_inline)) {
    const int i = lane & 3;
    const int32_t* src = lane < 4 ? bt_row + min((t + 2) * 4 + i, nbl - 1)
                         : VB     ? bt_row + min((t + 1) * 4 + i, nbl - 1)
                                  : exp_row + min(t, nkt - 1) * 4 + i;
    meta = *src;
  };

  // ---- wave w copies block w of a tile straight into LDS (1 KiB per
  // instruction): K from the pool (blocks past the table are left stale:
  // their keys are masked), V from the pool (VB) or from the fp16 copy in
  // the workspace (zero there past L).  `lane0` is the meta lane of block 0.
  auto copy_tile = [&](const char* src, char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::CP; ++i)
      __builtin_amdgcn_global_load_lds(src + i * 1024, (lds_void_t*)(dst + i * 1024), 16, 0, 0);
  };
  auto issue_k = [&](int kt, char* buf, int lane0) __attribute__((always_inline)) {
    if (kt * 4 + wave < nbl) {
      const int id = __builtin_amdgcn_readlane(meta, lane0 + wave);
      copy_tile(k_src + (size_t)id * p.block_bytes, buf + wave * S::TILE);
    }
  };
  auto issue_v = [&](int kt, char* buf, int lane0) __attribute__((always_inline)) {
    const int blk = kt * 4 + wave;
    if constexpr (VB) {
      if (blk < nbl) {
        const int id = __builtin_amdgcn_readlane(meta, lane0 + wave);
        copy_tile(v_src + (size_t)id * p.block_bytes, buf + wave * S::TILE);
      }
    } else {
      copy_tile(v_src + (size_t)blk * p.hkv * S::TILE, buf + wave * S::TILE);
    }
  };
  // VB: keys at or past L in the tile (unwritten slots of the last block,
  // stale LDS of blocks past the table) get a zero V, so that a zero
  // probability never meets a NaN.  Wave w clears its block's tail.
  auto clear_v_tail = [&](int kt, char* vbuf) __attribute__((always_inline)) {
    const int kb = kt * S::KT + wave * BS;         // first key of block `wave`
    const int t0 = max(0, min(BS, L - kb));        // its first invalid token
    if (t0 == BS) return;
    uint16_t* vt = reinterpret_cast<uint16_t*>(vbuf + wave * S::TILE);
    for (int d = lane; d < D; d += 64)
      for (int t = t0; t < BS; ++t) vt[((t >> 3) * D + d) * 8 + (t & 7)] = 0;
  };

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  // A finite floor keeps exp2(x - m) at 0 for masked x before any key is seen.
  float m_run = -1e30f;
  float l_run = 0.f;
  int kexp = 0;        // o counts in units of 2^kexp
  float corr = 1.f;    // rescale of o that the last softmax asked for
  bool resc = false;   // (deferred until the P.V products before it are issued)
  f32x16_t sc[2];      // S^T of the chunks of either parity
  uint32_t ph[2][8];   // their P: fp16 pairs (VB: the bf16 hi parts)
  uint32_t pl[2][8];   // VB: the bf16 lo parts

  // ---- building blocks of a 32-key chunk.  K operand: lane (h, r) reads key
  // pi(r) of the chunk; the 16 S^T values a lane then holds are keys
  // 16 (i / 8) + 8 h + i % 8 of the chunk, the k order of the P.V operands.
  const int pr = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
  auto k_frag = [&](const char* kbuf, int j, int ks) __attribute__((always_inline)) {
    const char* kp = kbuf + (2 * j + (r >> 4)) * S::TILE + (h * 16 + (pr & 15)) * 16;
    return *reinterpret_cast<const uint4*>(kp + ks * 512);
  };
  // V^T fragment i = kk * DB + db: block 2 j + kk, granule (key group h, d = 32 db + r)
  auto v_frag = [&](const char* vbuf, int j, int i) __attribute__((always_inline)) {
    const char* vp = vbuf + (2 * j + i / DB) * S::TILE + (h * D + r) * 16;
    return *reinterpret_cast<const uint4*>(vp + (i % DB) * 512);
  };
  auto qk_mfma = [&](uint4 a, int ks, f32x16_t& s) __attribute__((always_inline)) {
    const f32x16_t zero = {};
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qb[ks],
                                                ks == 0 ? zero : s, 0, 0, 0);
  };
  // P.V product i of a chunk: VB, i < 2 DB the hi and then the lo parts of P.
  auto pv_mfma = [&](uint4 v, int i, const uint32_t (&hi)[8], const uint32_t (&lo)[8]) __attribute__((always_inline)) {
    const int kk = (i / DB) & 1, db = i % DB;
    if constexpr (VB) {
      const uint32_t* w = i < 2 * DB ? hi : lo;
      const bf16x8_t pb = __builtin_bit_cast(
          bf16x8_t, make_uint4(w[4 * kk], w[4 * kk + 1], w[4 * kk + 2], w[4 * kk + 3]));
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v), pb, o[db], 0,
                                                      0, 0);
    } else {
      const f16x8_t pb = __builtin_bit_cast(
          f16x8_t, make_uint4(hi[4 * kk], hi[4 * kk + 1], hi[4 * kk + 2], hi[4 * kk + 3]));
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, v), pb, o[db], 0, 0,
                                                     0);
    }
  };
  // Softmax of a chunk in pieces: causal mask (chunks that reach the
  // diagonal), the chunk's row max, the running statistics, then P word w
  // (keys 2w, 2w + 1 of the lane's 16).
  auto sm_mask = [&](int ch, f32x16_t& s) __attribute__((always_inline)) {
    const int kl = lim - (32 * ch + 8 * h);  // offsets 16 (i / 8) + i % 8 up to kl are visible
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = (16 * (i >> 3) + (i & 7) <= kl) ? s[i] : -INFINITY;
  };
  auto sm_max = [&](const f32x16_t& s) __attribute__((always_inline)) {
    float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[0], s[1]),
                                            __builtin_elementwise_maximum(s[2], s[3]));
    float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[4], s[5]),
                                            __builtin_elementwise_maximum(s[6], s[7]));
    float d = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[8], s[9]),
                                            __builtin_elementwise_maximum(s[10], s[11]));
    float e = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[12], s[13]),
                                            __builtin_elementwise_maximum(s[14], s[15]));
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b),
                                         __builtin_elementwise_maximum(d, e));
  };
  // New running max only where it grew by more than the slack; the rescale
  // of o it implies waits for the next slot (P.V of the chunk before is in
  // flight), l is rescaled here.  Returns -m_run.
  auto sm_stats = [&](float mt) __attribute__((always_inline)) {
    mt = half_swap_max(mt) * c;
    const bool need = mt > m_run + kRescaleSlack;
    resc = __ballot(need) != 0;
    const float mnew = need ? mt : m_run;
    corr = __builtin_amdgcn_exp2f(m_run - mnew);
    l_run *= corr;
    m_run = mnew;
    return -m_run;
  };
  auto sm_word = [&](const f32x16_t& s, int w, float nm, uint32_t (&hi)[8], uint32_t (&lo)[8]) __attribute__((always_inline)) {
    const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w], c, nm));
    const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w + 1], c, nm));
    if constexpr (VB) {
      // P = hi + lo, both bf16 (16 significant bits together); V is bf16
      l_run += a + b;
      const bf16x2_t ab = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
      const uint32_t hw = __builtin_bit_cast(uint32_t, ab);
      hi[w] = hw;
      lo[w] = __builtin_bit_cast(
          uint32_t, __builtin_convertvector((f32x2_t){a - bf16_lo(hw), b - bf16_hi(hw)}, bf16x2_t));
    } else {
      // P in fp16; l sums the same rounded values that enter the product,
      // each fp16 half added to the fp32 sum by one v_fma_mix_f32 (x 1.0).
      // Not v_dot2: it waits while the matrix core of its SIMD is busy,
      // other VALU instructions do not.  The compiler makes a conversion
      // and an add of each half, hence the asm.
      hi[w] = pack_f16x2(a, b);
      asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]" : "+v"(l_run) : "v"(hi[w]));
      asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(l_run) : "v"(hi[w]));
    }
  };
  auto rescale_o = [&](float f) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= f;
  };

  // ---- slot ch of the pipeline: S^T of chunk ch + 1 (MFMA), the softmax of
  // chunk ch (VALU) and O^T += V^T P^T of chunk ch - 1 (MFMA).  The three are
  // independent, so the softmax runs while the matrix core works.  The K of
  // chunk ch + 1 and the V of chunk ch - 1 are chunk j of `kbuf` and `vbuf`.
  constexpr int R = PVN / KS;  // P.V products per QK product in the interleave
  static_assert(R * KS == PVN, "interleave shape");
  auto slot_fast = [&](int ch, const char* kbuf, const char* vbuf, int j, const f32x16_t& s_in,
                       f32x16_t& s_out, const uint32_t (&hin)[8], const uint32_t (&lin)[8],
                       uint32_t (&hout)[8], uint32_t (&lout)[8]) __attribute__((always_inline)) {
    // fragments in the order the products consume them, LA groups ahead
    constexpr int LA = 2;
    uint4 a[KS], v[2 * DB];
    auto read_group = [&](int g) __attribute__((always_inline)) {
      a[g] = k_frag(kbuf, j, g);
#pragma unroll
      for (int u = 0; u < R; ++u)
        if (g * R + u < 2 * DB) v[g * R + u] = v_frag(vbuf, j, g * R + u);
    };
#pragma unroll
    for (int g = 0; g < LA; ++g) read_group(g);
    __builtin_amdgcn_sched_barrier(0);
    float mt = 0.f, nm = 0.f;
#pragma unroll
    for (int g = 0; g < KS; ++g) {
      if (g + LA < KS) read_group(g + LA);
      qk_mfma(a[g], g, s_out);
#pragma unroll
      for (int u = 0; u < R; ++u) pv_mfma(v[(g * R + u) % (2 * DB)], g * R + u, hin, lin);
      if (g == 0) mt = sm_max(s_in);
      if (g == 1) nm = sm_stats(mt);
      if (g >= 2) {
#pragma unroll
        for (int w = (g - 2) * 8 / (KS - 2); w < (g - 1) * 8 / (KS - 2); ++w)
          sm_word(s_in, w, nm, hout, lout);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Slots at the ends of a wave's chunks and chunks on the diagonal: the
  // same work in sequence, each part only where it applies.
  auto slot_gen = [&](int ch, const char* kbuf, const char* vbuf, int j, f32x16_t& s_in,
                      f32x16_t& s_out, const uint32_t (&hin)[8], const uint32_t (&lin)[8],
                      uint32_t (&hout)[8], uint32_t (&lout)[8]) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if (ch > c_beg && ch <= c_end) {  // P.V of chunk ch - 1
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint4 v[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) v[db] = v_frag(vbuf, j, kk * DB + db);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          pv_mfma(v[db], kk * DB + db, hin, lin);
          if constexpr (VB) pv_mfma(v[db], 2 * DB + kk * DB + db, hin, lin);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ch + 1 < c_end) {  // S^T of chunk ch + 1
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qk_mfma(k_frag(kbuf, j, ks), ks, s_out);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ch < c_end) {  // softmax of chunk ch
      if (uniform(32 * ch + 31 > wp0)) sm_mask(ch, s_in);
      const float nm = sm_stats(sm_max(s_in));
#pragma unroll
      for (int w = 0; w < 8; ++w) sm_word(s_in, w, nm, hout, lout);
    }
  };
  // Before the P.V products of chunk ch - 1: the rescale of o the last
  // softmax asked for, and (fp16 V copies) the power-of-two exponents e0, e1
  // of its two blocks.  With E the largest of kexp, e0, e1, o moves to units
  // of 2^E and block k's probabilities are scaled by 2^(ek - E), so that both
  // blocks' products land in o's units.  Only tiles with some |v| >= 2^16
  // have an exponent other than 0.
  auto pre_slot = [&](int ch, int e0, int e1, uint32_t (&hin)[8]) __attribute__((always_inline)) {
    if (uniform(resc)) {
      rescale_o(corr);
      resc = false;
    }
    if constexpr (!VB) {
      if (uniform(ch > c_beg && ch <= c_end && (e0 != kexp || e1 != kexp))) {
        const int E = max(kexp, max(e0, e1));
        if (E > kexp) rescale_o(__builtin_ldexpf(1.f, kexp - E));
        const int ek[2] = {e0, e1};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const _Float16 f = (_Float16)__builtin_ldexpf(1.f, ek[kk] - E);
          const f16x2_t f2 = {f, f};
#pragma unroll
          for (int w = 4 * kk; w < 4 * kk + 4; ++w)
            hin[w] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, hin[w]) * f2);
        }
        kexp = uniform(E);
      }
    }
  };

  // vmcnt(0) with the other counters left alone (gfx9 s_waitcnt encoding)
  constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);
  // Iteration t: K of tile t + 1 and V of tile t are in `kcur` and `vcur`;
  // it starts the copies of K(t + 2) into `knext` (K(t) is done) and of
  // V(t + 1) into `vnext` (V(t - 1) is done), then runs slots 2t + 1, 2t + 2.
  // FAST: both slots have all three parts and no diagonal chunk.
  auto iter = [&](auto fast_tag, int t, const char* kcur, char* vcur, char* knext, char* vnext)
      __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_tag)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies have landed
    __syncthreads();                       // everyone's have, and every read of the old tiles is done
    if constexpr (VB) {
      if (t * S::KT + S::KT > L) {         // uniform: the tile reaches past the last key
        clear_v_tail(t, vcur);
        __syncthreads();
      }
    }
    int ex[4] = {0, 0, 0, 0};
    if constexpr (!VB) {
      ex[0] = __builtin_amdgcn_readlane(meta, 4);
      ex[1] = __builtin_amdgcn_readlane(meta, 5);
      ex[2] = __builtin_amdgcn_readlane(meta, 6);
      ex[3] = __builtin_amdgcn_readlane(meta, 7);
    }
    if (t + 2 < te) issue_k(t + 2, knext, 0);
    if (t + 1 < te) issue_v(t + 1, vnext, 4);
    load_meta(t + 1);
    pre_slot(2 * t + 1, ex[0], ex[1], ph[0]);
    if constexpr (FAST)
      slot_fast(2 * t + 1, kcur, vcur, 0, sc[1], sc[0], ph[0], pl[0], ph[1], pl[1]);
    else
      slot_gen(2 * t + 1, kcur, vcur, 0, sc[1], sc[0], ph[0], pl[0], ph[1], pl[1]);
    pre_slot(2 * t + 2, ex[2], ex[3], ph[1]);
    if constexpr (FAST)
      slot_fast(2 * t + 2, kcur, vcur, 1, sc[0], sc[1], ph[1], pl[1], ph[0], pl[0]);
    else
      slot_gen(2 * t + 2, kcur, vcur, 1, sc[0], sc[1], ph[1], pl[1], ph[0], pl[0]);
  };
  using Fast = std::true_type;
  using Gen = std::false_type;

  __builtin_amdgcn_s_waitcnt(kWaitVm0);    // ids of tiles tb and tb + 1
  if (tb < te) {
    issue_k(tb, kb0, 0);
    issue_v(tb, vb0, 0);
  }
  if (tb + 1 < te) issue_k(tb + 1, kb1, 4);
  load_meta(tb);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (c_end > c_beg) {  // S^T of chunk c_beg, then slot c_beg
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qk_mfma(k_frag(kb0, 0, ks), ks, sc[0]);
  }
  slot_gen(c_beg, kb0, vb0, 1, sc[0], sc[1], ph[1], pl[1], ph[0], pl[0]);
  // Leading iterations whose slots are all fast (chunk 2t + 3 exists and
  // chunk 2t + 2 ends at or before the wave's first row), then the rest.
  // Two loops rather than one with a branch per slot: the compiler would keep
  // both sides' accumulators alive across such a branch.  Buffers alternate
  // with the iteration's parity counted from tb.
  const int n_a = max(0, (c_end - 2) / 2 - tb);
  const int n_b = wp0 >= 95 ? max(0, (wp0 - 95) / 64 + 1 - tb) : 0;
  const int nfast = uniform(min(min(n_a, n_b), te - tb));
  for (int u = 0; u < nfast; u += 2) {
    iter(Fast{}, tb + u, kb1, vb0, kb0, vb1);
    if (u + 1 < nfast) iter(Fast{}, tb + u + 1, kb0, vb1, kb1, vb0);
  }
  for (int u = nfast; u < niter; ++u) {
    const bool odd = u & 1;
    iter(Gen{}, tb + u, odd ? kb0 : kb1, odd ? vb1 : vb0, odd ? kb1 : kb0, odd ? vb0 : vb1);
  }

  if constexpr (SPLIT) {
    // Every tile read of both groups is done; group 1's state goes through
    // LDS (lane-major 16-byte quads: conflict-free) to group 0.
    __syncthreads();
    float* mo = reinterpret_cast<float*>(wave < 2 ? xo0 : xo1) + (wave & 1) * (DB * 16 * 64);
    float* ml = reinterpret_cast<float*>(xml) + wave * 3 * 64;
    if (grp) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<float4*>(mo + ((db * 4 + i4) * 64 + lane) * 4) =
              make_float4(o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]);
      ml[lane] = m_run;
      ml[64 + lane] = l_run;
      ml[128 + lane] = __int_as_float(kexp);
    }
    __syncthreads();
    if (grp) return;
    // Both parts relative to the larger max M, o in units of 2^K with K the
    // larger exponent.  A part that saw no key has m = -1e30 and weight 0.
    const float m1 = ml[lane], l1 = ml[64 + lane];
    const int k1 = uniform(__float_as_int(ml[128 + lane]));
    const float mm = fmaxf(m_run, m1);
    const float f0 = __builtin_amdgcn_exp2f(m_run - mm), f1 = __builtin_amdgcn_exp2f(m1 - mm);
    l_run = l_run * f0 + l1 * f1;
    const int kk = max(kexp, k1);
    const float a0 = f0 * __builtin_ldexpf(1.f, kexp - kk);
    const float a1 = f1 * __builtin_ldexpf(1.f, k1 - kk);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 b = *reinterpret_cast<const float4*>(mo + ((db * 4 + i4) * 64 + lane) * 4);
        o[db][4 * i4] = o[db][4 * i4] * a0 + b.x * a1;
        o[db][4 * i4 + 1] = o[db][4 * i4 + 1] * a0 + b.y * a1;
        o[db][4 * i4 + 2] = o[db][4 * i4 + 2] * a0 + b.z * a1;
        o[db][4 * i4 + 3] = o[db][4 * i4 + 3] * a0 + b.w * a1;
      }
    kexp = kk;
  }

  const float l_tot = half_swap_sum(l_run);
  if (row_ok) {
    float* orow = p.out + (((size_t)row0 + (my_pos - qfirst)) * hq + head) * D;
    const float inv = __builtin_ldexpf(1.f / l_tot, kexp);
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * h;
        *reinterpret_cast<float4*>(orow + d) =
            make_float4(o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv, o[db][4 * i4 + 2] * inv,
                        o[db][4 * i4 + 3] * inv);
      }
    }
  }
}

template <int D, int G, bool VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill_tile(
    PrefillParams p) {
  constexpr int BUF = PrefillShape<D, G>::BUF;
  __shared__ __align__(16) char kb0[BUF];
  __shared__ __align__(16) char kb1[BUF];
  __shared__ __align__(16) char vb0[BUF];
  __shared__ __align__(16) char vb1[BUF];
  if (p.prio) __builtin_amdgcn_s_setprio(3);
  prefill_item<D, G, VB>(p, blockIdx.x, kb0, kb1, vb0, vb1);
}

// The fp16-V tile kernel with each item's key tiles split between two groups
// of 4 waves (see prefill_item): one 8-wave workgroup of 128 KiB LDS per CU,
// so two waves per SIMD on every item.  For calls whose items each get a CU
// of their own; a 4-wave workgroup alone on a CU has one wave per SIMD.
// With more items than CUs, k_prefill_tile's two workgroups per CU overlap
// each other's start and end, which this kernel pays per item.
template <int D, int G>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill_split(
    PrefillParams p) {
  constexpr int BUF = PrefillShape<D, G>::BUF;
  static_assert(2 * BUF >= 2 * (D / 32) * 16 * 64 * 4, "two waves' O fit in one K buffer pair");
  __shared__ __align__(16) char kb0[2][BUF];
  __shared__ __align__(16) char kb1[2][BUF];
  __shared__ __align__(16) char vb0[2][BUF];
  __shared__ __align__(16) char vb1[2][BUF];
  const int grp = uniform((int)threadIdx.x >> 8);
  prefill_item<D, G, false, true>(p, blockIdx.x, kb0[grp], kb1[grp], vb0[grp], vb1[grp], grp,
                                  &kb0[0][0], &kb1[0][0], &vb0[0][0]);
}

// ---- Multi-query rows: pure prefill calls whose sequences all have at most
// 32 / G query rows (speculative verify, short chunks).  One workgroup per
// (sequence, kv head).  The 32 rows of every MFMA are the G query heads x
// 32 / G positions, so no row is padding; wave w takes the sequence's 32-key
// chunks w, w + 4, w + 8, ... with K and V read straight from the pool into
// MFMA operand registers (no LDS, no barrier), and the four waves' partial
// (max, sum, O) are merged through LDS at the end.  Operand and accumulator
// layouts are those of k_prefill_tile's bf16-V variant: lane (h, r) of the
// K operand reads key pi(r), pi swapping bits 2 and 3, so that the 16 S^T
// values a lane holds are the keys 16 (i / 8) + 8 h + i % 8 that the P.V
// operand needs; P enters as a bf16 hi + lo pair.
// Sequences in the order their workgroups start: longest first, so that the
// long ones do not start in the last round.  n = 0: index order.
constexpr int kMqOrderMax = 1024;
struct MqParams {
  PrefillParams p;
  int n;
  uint16_t order[kMqOrderMax];
};

template <int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill_mq(
    MqParams mp) {
  const PrefillParams& p = mp.p;
  constexpr int NP = 32 / G;        // positions per wave
  constexpr int KS = D / 16;        // MFMA k-steps over the head dim
  constexpr int DB = D / 32;        // 32-row d blocks of O^T
  constexpr int TILE = BS * D * 2;  // bytes of one block's K (or V) tile
  __shared__ float mg_o[4][DB * 16][64];
  __shared__ float mg_ml[4][2][64];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int kvh = blockIdx.x % p.hkv;
  const int rank = blockIdx.x / p.hkv;
  const int s = mp.n > 0 ? (int)mp.order[rank] : rank;
  const int hq = p.hkv * G;
  const int L = uniform(p.seq_lens[s]);
  const int row0 = uniform(p.qsl[s]);
  const int ql = uniform(p.qsl[s + 1]) - row0;
  if (ql <= 0) return;                   // uniform over the workgroup
  const int qfirst = L - ql;
  const int h = lane >> 5;
  const int r = lane & 31;
  const int g = r / NP, i = r % NP;      // this lane's query row: head g, position i
  const bool row_ok = i < ql;
  const int lim = row_ok ? qfirst + i : -1;  // last key the row sees
  const int head = kvh * G + g;
  const bool neg = p.scale_log2 < 0.f;
  const float c = fmaxf(fabsf(p.scale_log2), 1.17549435e-38f);

  // Q^T operand: lane (h, r) holds q[row r][16 ks + 8 h .. + 8]; a negative
  // scale is carried by negating q (exact), so that c > 0.
  bf16x8_t qb[KS];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(
        p.q + ((size_t)(row0 + (row_ok ? i : 0)) * hq + head) * D);
    const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = row_ok ? qrow[2 * ks + h] : make_uint4(0, 0, 0, 0);
      v.x ^= flip; v.y ^= flip; v.z ^= flip; v.w ^= flip;
      qb[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int k = 0; k < 16; ++k) o[db][k] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  const int pr = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
  const int nbl = (L + BS - 1) / BS;
  const int nch = (L + 31) / 32;
  const int32_t* bt_row = p.block_tables + (size_t)s * p.max_blocks;
  const char* kbase = p.kv + (size_t)kvh * 2 * TILE;
  const char* vbase = kbase + TILE;

  // K and V operands of one chunk; two sets alternate so that the next
  // chunk's loads are in flight while this one is computed.
  struct ChunkRegs {
    uint4 a[KS];      // K operand of key pi(r), d-granule 2 ks + h
    uint4 v[2][DB];   // V^T operand of block kk: granule (key group h, d = 32 db + r)
  };
  // Block ids of chunk ch (clamped to the last valid entry past the table's
  // end: those keys are masked and their V zeroed).
  auto chunk_ids = [&](int ch, int& b0, int& b1) __attribute__((always_inline)) {
    const int e = min(2 * ch, nbl - 1);
    b0 = uniform(bt_row[e]);
    b1 = uniform(bt_row[min(e + 1, nbl - 1)]);
  };
  auto load_chunk = [&](ChunkRegs& cr, int b0, int b1) __attribute__((always_inline)) {
    const char* kp = kbase + (size_t)((pr >> 4) ? b1 : b0) * p.block_bytes + (h * 16 + (pr & 15)) * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cr.a[ks] = load_once(kp + ks * 512);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char* vp = vbase + (size_t)(kk ? b1 : b0) * p.block_bytes + (h * D + r) * 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) cr.v[kk][db] = load_once(vp + db * 512);
    }
  };
  auto compute_chunk = [&](ChunkRegs& cr, int ch) __attribute__((always_inline)) {
    f32x16_t sacc;
#pragma unroll
    for (int k = 0; k < 16; ++k) sacc[k] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cr.a[ks]), qb[ks],
                                                     sacc, 0, 0, 0);
    const int kj = 32 * ch;
    if (uniform(kj + 31 > qfirst)) {  // the chunk reaches the first row's position (or L)
      const int kl = lim - (kj + 8 * h);
#pragma unroll
      for (int k = 0; k < 16; ++k) sacc[k] = (16 * (k >> 3) + (k & 7) <= kl) ? sacc[k] : -INFINITY;
      // keys at or past L (unwritten slots, blocks past the table) get a zero
      // V, so that a zero probability never meets a NaN
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int t0 = L - (kj + 16 * kk + 8 * h);  // keys of this granule from t0 on are past L
        if (t0 < 8) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            uint32_t w4[4] = {cr.v[kk][db].x, cr.v[kk][db].y, cr.v[kk][db].z, cr.v[kk][db].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= t0) w4[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            cr.v[kk][db] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
          }
        }
      }
    }
    float mt = sacc[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) mt = __builtin_elementwise_maximum(mt, sacc[k]);
    mt = half_swap_max(mt) * c;
    if (mt > m_run + kRescaleSlack) {  // per lane; the rows of a wave rescale on their own
      const float corr = __builtin_amdgcn_exp2f(m_run - mt);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int k = 0; k < 16; ++k) o[db][k] *= corr;
      m_run = mt;
    }
    const float nm = -m_run;
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int w2 = 0; w2 < 8; ++w2) {
      const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * w2], c, nm));
      const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * w2 + 1], c, nm));
      l_run += x0 + x1;
      const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));
      ph[w2] = hw;
      pl[w2] = __builtin_bit_cast(
          uint32_t, __builtin_convertvector((f32x2_t){x0 - bf16_lo(hw), x1 - bf16_hi(hw)}, bf16x2_t));
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8_t bh = __builtin_bit_cast(
          bf16x8_t, make_uint4(ph[4 * kk], ph[4 * kk + 1], ph[4 * kk + 2], ph[4 * kk + 3]));
      const bf16x8_t bl = __builtin_bit_cast(
          bf16x8_t, make_uint4(pl[4 * kk], pl[4 * kk + 1], pl[4 * kk + 2], pl[4 * kk + 3]));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, cr.v[kk][db]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, bh, o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, bl, o[db], 0, 0, 0);
      }
    }
  };

  // Chunks wave, wave + 4, ...: chunk k + 1's K/V and chunk k + 2's block ids
  // are requested before chunk k is computed.  Past the wave's last chunk the
  // loads repeat its last blocks (cache hits) instead of branching around
  // them, so every iteration issues the same loads.
  if (wave < nch) {
    ChunkRegs ra, rb;
    int b0, b1, n0, n1;
    chunk_ids(wave, b0, b1);
    load_chunk(ra, b0, b1);
    chunk_ids(min(wave + 4, nch - 1), n0, n1);
    for (int ch = wave; ch < nch; ch += 8) {
      load_chunk(rb, n0, n1);
      chunk_ids(min(ch + 8, nch - 1), b0, b1);
      compute_chunk(ra, ch);
      if (ch + 4 >= nch) break;
      load_chunk(ra, b0, b1);
      chunk_ids(min(ch + 12, nch - 1), n0, n1);
      compute_chunk(rb, ch + 4);
    }
  }

  // ---- merge the four waves' partials: wave w writes its own, then forms
  // the output of d-block w (lane (h, r): row r, d = 32 w + 8 i4 + 4 h .. + 4)
  const float l_tot = half_swap_sum(l_run);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int k = 0; k < 16; ++k) mg_o[wave][db * 16 + k][lane] = o[db][k];
  mg_ml[wave][0][lane] = m_run;
  mg_ml[wave][1][lane] = l_tot;
  __syncthreads();
  if (wave >= DB || !row_ok) return;
  float M = -INFINITY;
#pragma unroll
  for (int sw = 0; sw < 4; ++sw) M = fmaxf(M, mg_ml[sw][0][lane]);
  float den = 0.f, num[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) num[k] = 0.f;
#pragma unroll
  for (int sw = 0; sw < 4; ++sw) {
    const float a = __builtin_amdgcn_exp2f(mg_ml[sw][0][lane] - M);
    den = fmaf(a, mg_ml[sw][1][lane], den);
#pragma unroll
    for (int k = 0; k < 16; ++k) num[k] = fmaf(a, mg_o[sw][wave * 16 + k][lane], num[k]);
  }
  const float inv = 1.f / den;
  float* orow = p.out + (((size_t)row0 + i) * hq + head) * D;
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int d = 32 * wave + 8 * i4 + 4 * h;
    *reinterpret_cast<float4*>(orow + d) =
        make_float4(num[4 * i4] * inv, num[4 * i4 + 1] * inv, num[4 * i4 + 2] * inv,
                    num[4 * i4 + 3] * inv);
  }
}

// One launch for a mixed batch (PKV_MIXED=fused): workgroups [0, n_prefill)
// run prefill tiles (compute-bound, MFMA) and the rest run four decode items
// each, one per wave (bandwidth-bound).  Every workgroup holds the prefill
// tiles' 64 KiB of LDS, so the decode workgroups mostly follow the prefill
// ones; the default mixed path runs the two kinds of work side by side on
// two streams instead (mixed_concurrent).
struct MixedParams {
  PrefillParams pp;
  DecodeParams dp;
  int n_prefill;
};

template <int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_mixed(MixedParams m) {
  constexpr int DEC = DecodeLds<2, D, G>::BYTES;
  constexpr int BUF = PrefillShape<D, G>::BUF;
  static_assert(2 * DEC <= BUF, "two decode waves share one prefill buffer");
  __shared__ __align__(16) char kb0[BUF];
  __shared__ __align__(16) char kb1[BUF];
  __shared__ __align__(16) char vb0[BUF];
  __shared__ __align__(16) char vb1[BUF];
  if ((int)blockIdx.x < m.n_prefill) {
    prefill_item<D, G, false>(m.pp, blockIdx.x, kb0, kb1, vb0, vb1);
  } else {
    const int wave = threadIdx.x >> 6;
    const int item = ((int)blockIdx.x - m.n_prefill) * 4 + wave;
    decode_item<2, D, G>(m.dp, item, (wave < 2 ? kb0 : kb1) + (wave & 1) * DEC);
  }
}

template <int D>
static hipError_t v_fp16(const PrefillParams& p, hipStream_t stream) {
  const int64_t items = p.vblocks * p.hkv;
  hipLaunchKernelGGL((k_v_fp16<D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// `lds_pad`: extra LDS bytes per 4-wave workgroup (limits how many share a CU).
template <int D, bool VB>
static hipError_t prefill_g(int G, const PrefillParams& p, int64_t grid, bool split,
                            hipStream_t stream, size_t lds_pad = 0) {
  if constexpr (!VB) {
    if (hipError_t e = v_fp16<D>(p, stream)) return e;
    if (split) {
      PrefillParams ps = p;
      ps.pair_from = 0;  // one workgroup per CU: the dispatcher balances
      const dim3 g((unsigned)grid), b(512);
      switch (G) {
        case 1: hipLaunchKernelGGL((k_prefill_split<D, 1>), g, b, 0, stream, ps); break;
        case 2: hipLaunchKernelGGL((k_prefill_split<D, 2>), g, b, 0, stream, ps); break;
        case 4: hipLaunchKernelGGL((k_prefill_split<D, 4>), g, b, 0, stream, ps); break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
  }
  const dim3 g((unsigned)grid), b(256);
  const unsigned pad = (unsigned)lds_pad;
  switch (G) {
    case 1: hipLaunchKernelGGL((k_prefill_tile<D, 1, VB>), g, b, pad, stream, p); break;
    case 2: hipLaunchKernelGGL((k_prefill_tile<D, 2, VB>), g, b, pad, stream, p); break;
    case 4: hipLaunchKernelGGL((k_prefill_tile<D, 4, VB>), g, b, pad, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

static PrefillParams make_prefill_params(const CacheDesc& c, const AttnDesc& a) {
  PrefillParams p;
  p.kv = c.kv;
  p.block_bytes = c.block_bytes;
  p.hkv = c.hkv;
  p.q = static_cast<const uint16_t*>(a.q);
  p.out = a.out;
  p.block_tables = a.block_tables;
  p.max_blocks = a.max_blocks;
  p.seq_lens = a.seq_lens;
  p.qsl = a.query_start_loc;
  p.num_seqs = a.num_seqs;
  p.scale_log2 = a.scale * kLog2e;
  p.vh = a.ws_v;
  p.vexp = a.ws_vexp;
  p.vblocks = a.prefill_vblocks;
  p.items = (int)a.prefill_tiles;
  // Pair heavy with light items on a CU when the prefill workgroups fill at
  // most two rounds of the CUs (more rounds are balanced by the dispatcher).
  p.pair_from = 0;
  p.prio = 0;
  const int cus = device_cus();
  if (cus > 0) {
    const int64_t round_items = cus / c.hkv;
    if (round_items > 0 && a.prefill_tiles > round_items && a.prefill_tiles <= 2 * round_items)
      p.pair_from = (int)round_items;
  }
  return p;
}

template <int D>
static hipError_t prefill_mq(int G, const MqParams& mp, int64_t grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((k_prefill_mq<D, 1>), g, b, 0, stream, mp); break;
    case 2: hipLaunchKernelGGL((k_prefill_mq<D, 2>), g, b, 0, stream, mp); break;
    case 4: hipLaunchKernelGGL((k_prefill_mq<D, 4>), g, b, 0, stream, mp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_rows(const CacheDesc& c, const AttnDesc& a, hipStream_t stream) {
  if (a.prefill_tiles == 0) return hipSuccess;
  if (c.dtype_bytes != 2) return hipErrorInvalidValue;
  const PrefillParams p = make_prefill_params(c, a);
  const int G = a.hq / c.hkv;
  if (a.prefill_mq) {  // every sequence has at most 32 / G query rows
    MqParams mp;
    mp.p = p;
    mp.n = 0;
    if (a.h_seq_lens && a.num_seqs <= kMqOrderMax) {  // longest sequences start first
      for (int i = 0; i < a.num_seqs; ++i) mp.order[i] = (uint16_t)i;
      std::stable_sort(mp.order, mp.order + a.num_seqs, [&a](uint16_t x, uint16_t y) {
        return a.h_seq_lens[x] > a.h_seq_lens[y];
      });
      mp.n = a.num_seqs;
    }
    const int64_t grid = (int64_t)a.num_seqs * c.hkv;
    if (c.head_size == 128) return prefill_mq<128>(G, mp, grid, stream);
    if (c.head_size == 64) return prefill_mq<64>(G, mp, grid, stream);
    return hipErrorInvalidValue;
  }
  const int64_t grid = a.prefill_tiles * c.hkv;
  const int cus = device_cus();
  const bool split = a.prefill_split > 0 || (a.prefill_split < 0 && cus > 0 && grid <= cus);
  if (a.prefill_v_bf16) {
    if (c.head_size == 128) return prefill_g<128, true>(G, p, grid, split, stream);
    if (c.head_size == 64) return prefill_g<64, true>(G, p, grid, split, stream);
  } else {
    if (c.head_size == 128) return prefill_g<128, false>(G, p, grid, split, stream);
    if (c.head_size == 64) return prefill_g<64, false>(G, p, grid, split, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, int G>
static hipError_t mixed_t(const MixedParams& m, int64_t grid, int num_seqs, int hkv,
                          hipStream_t stream) {
  if (hipError_t e = v_fp16<D>(m.pp, stream)) return e;
  hipLaunchKernelGGL((k_mixed<D, G>), dim3((unsigned)grid), dim3(256), 0, stream, m);
  hipLaunchKernelGGL((k_decode_merge<D, G>), dim3((unsigned)((int64_t)num_seqs * hkv)),
                     dim3(64 * (G < 4 ? G : 4)), 0, stream, m.dp);
  return hipGetLastError();
}

// The library's side stream of a device, with the events that fork work
// onto it from a caller's stream and join it back.  Created on first use
// (default priority, non-blocking) and kept until the process ends.  The
// mutex keeps one call's record / wait pairs together when host threads
// call at once.
struct SideStream {
  std::once_flag once;
  hipError_t err = hipSuccess;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
constexpr int kMaxDevices = 64;
static SideStream g_side[kMaxDevices];

static SideStream* side_stream(hipError_t* err) {
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  SideStream& ss = g_side[dev];
  std::call_once(ss.once, [&ss]() {
    ss.err = hipStreamCreateWithFlags(&ss.side, hipStreamNonBlocking);
    if (ss.err == hipSuccess) ss.err = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (ss.err == hipSuccess) ss.err = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
  });
  *err = ss.err;
  return ss.err == hipSuccess ? &ss : nullptr;
}

// Scratch of paged_attention_decode_noalloc: the stream decode's partials
// and counters in a fixed array of device memory that the code object holds
// on every device it runs on, until the process ends, so that entry point
// allocates nothing.  In host code the array's name is not its device
// address: the address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address reaches a kernel.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

struct ScratchAddr {
  std::once_flag once;
  hipError_t err = hipSuccess;
  char* ptr = nullptr;
};
static ScratchAddr g_scratch[kMaxDevices];

hipError_t noalloc_scratch(char** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchAddr& sa = g_scratch[dev];
  std::call_once(sa.once, [&sa]() {
    void* addr = nullptr;
    sa.err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (sa.err == hipSuccess && !addr) sa.err = hipErrorInvalidSymbol;
    if (sa.err == hipSuccess) sa.ptr = static_cast<char*>(addr);
  });
  *ptr = sa.ptr;
  return sa.err;
}

// Prefill tiles (HBM-light, MFMA-bound) and decode rows (HBM-bound) of one
// mixed call side by side: the fp16 copy of V and then the tiles on the
// side stream, the stream decode on the caller's.  The tile kernel gets ~81
// KiB of LDS per workgroup, so one shares a CU (one wave per SIMD, ~200
// VGPRs); the stream decode runs one wave per SIMD (~220 VGPRs), and both
// fit a SIMD's 512.  The prefill waves take the higher issue priority: the
// decode waves mostly wait for memory.
static hipError_t mixed_concurrent(const CacheDesc& c, const AttnDesc& a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  SideStream* ss = side_stream(&e);
  if (!ss) return e;
  PrefillParams p = make_prefill_params(c, a);
  p.pair_from = 0;  // one workgroup per CU: heaviest first, the dispatcher balances
  p.prio = 1;
  const int G = a.hq / c.hkv;
  const int64_t grid = a.prefill_tiles * c.hkv;
  constexpr size_t kCuLds = 160 * 1024;
  if (c.head_size != 128 && c.head_size != 64) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(ss->mu);
  if ((e = hipEventRecord(ss->fork, stream))) return e;
  if ((e = hipStreamWaitEvent(ss->side, ss->fork, 0))) return e;
  // Once forked, the side stream is always joined back, also when a launch
  // failed, so nothing of this call runs unordered with the caller's stream.
  if (c.head_size == 128)
    e = prefill_g<128, false>(G, p, grid, false, ss->side,
                              kCuLds / 2 + 1024 - PrefillShape<128, 4>::BUF * 4);
  else
    e = prefill_g<64, false>(G, p, grid, false, ss->side,
                             kCuLds / 2 + 1024 - PrefillShape<64, 4>::BUF * 4);
  const hipError_t e_dec = e ? hipSuccess : launch_decode_stream(c, a, stream);
  hipError_t e_join = hipEventRecord(ss->join, ss->side);
  if (e_join == hipSuccess) e_join = hipStreamWaitEvent(stream, ss->join, 0);
  return e ? e : e_dec ? e_dec : e_join;
}

hipError_t launch_mixed_rows(const CacheDesc& c, const AttnDesc& a, hipStream_t stream) {
  if (c.dtype_bytes != 2) return hipErrorInvalidValue;
  if (a.stream_waves > 0) return mixed_concurrent(c, a, stream);
  MixedParams m;
  m.pp = make_prefill_params(c, a);
  m.dp = make_decode_params(c, a);
  m.n_prefill = (int)(a.prefill_tiles * c.hkv);
  const int64_t decode_wgs = (a.decode_units * c.hkv + 3) / 4;
  const int64_t grid = m.n_prefill + decode_wgs;
  const int G = a.hq / c.hkv;
  if (c.head_size == 128) {
    switch (G) {
      case 1: return mixed_t<128, 1>(m, grid, a.num_seqs, c.hkv, stream);
      case 2: return mixed_t<128, 2>(m, grid, a.num_seqs, c.hkv, stream);
      case 4: return mixed_t<128, 4>(m, grid, a.num_seqs, c.hkv, stream);
    }
  } else if (c.head_size == 64) {
    switch (G) {
      case 1: return mixed_t<64, 1>(m, grid, a.num_seqs, c.hkv, stream);
      case 2: return mixed_t<64, 2>(m, grid, a.num_seqs, c.hkv, stream);
      case 4: return mixed_t<64, 4>(m, grid, a.num_seqs, c.hkv, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
