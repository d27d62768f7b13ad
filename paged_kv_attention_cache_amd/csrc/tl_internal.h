// Internal declarations of libtl: device helpers shared by the kernels and the
// host launchers that tl_api.hip calls after validating arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tl.h"

namespace tl {

// ------------------------------------------------------------ vector types
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2, KV_FP8U = 3, KV_INT8 = 4 };
constexpr bool kv_fp8(int k) { return k == KV_FP8 || k == KV_FP8U; }      // e4m3fn codes
constexpr bool kv_scaled(int k) { return k == KV_FP8 || k == KV_INT8; }   // with (token, head) scales

template <int KVT> struct KvTraits;
template <> struct KvTraits<KV_F32> { typedef float T; static constexpr int BYTES = 4; static constexpr int X = 4; };
template <> struct KvTraits<KV_BF16> { typedef uint16_t T; static constexpr int BYTES = 2; static constexpr int X = 8; };
template <> struct KvTraits<KV_FP8> { typedef uint8_t T; static constexpr int BYTES = 1; static constexpr int X = 16; };
template <> struct KvTraits<KV_FP8U> : KvTraits<KV_FP8> {};
template <> struct KvTraits<KV_INT8> : KvTraits<KV_FP8> {};

constexpr float LOG2E = 1.4426950408889634f;
constexpr int KEY_BLOCK = 2048;  // the pages' key-block width; loop bounds are taken per block

// ----------------------------------------------------------- conversions
// bf16 bits -> f32: the bf16 pattern is the top half of the f32 pattern (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// four fp8 e4m3fn codes packed in a dword -> four f32 (hardware convert, exact)
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// four int8 codes packed in a dword -> four f32 (exact)
__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (float)(int8_t)(w >> (8 * i));  // sign-extended byte i
}

// widen one 16-byte chunk of stored elements to f32 (X values)
template <int KVT>
__device__ __forceinline__ void widen_chunk(const uint4& c, float* o) {
  if constexpr (KVT == KV_F32) {
    o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y);
    o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
  } else if constexpr (KVT == KV_BF16) {
    o[0] = bf16_lo(c.x); o[1] = bf16_hi(c.x); o[2] = bf16_lo(c.y); o[3] = bf16_hi(c.y);
    o[4] = bf16_lo(c.z); o[5] = bf16_hi(c.z); o[6] = bf16_lo(c.w); o[7] = bf16_hi(c.w);
  } else if constexpr (KVT == KV_INT8) {
    i8x4_to_f32(c.x, o); i8x4_to_f32(c.y, o + 4); i8x4_to_f32(c.z, o + 8); i8x4_to_f32(c.w, o + 12);
  } else {
    fp8x4_to_f32(c.x, o); fp8x4_to_f32(c.y, o + 4); fp8x4_to_f32(c.z, o + 8); fp8x4_to_f32(c.w, o + 12);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load marked nontemporal: data read once (the KV pages of a decode step)
// stream through the caches without displacing other lines, which also sustains a
// higher HBM read rate than plain loads.
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 x = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// broadcast lane (lane & ~3) | R of each quad to the whole quad (DPP quad_perm)
template <int R>
__device__ __forceinline__ float quad_bcast(float v) {
  constexpr int ctrl = R | (R << 2) | (R << 4) | (R << 6);
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }
__device__ __forceinline__ float wave_xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

// ------------------------------------------------------------ launch args
struct PoolArgs {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  int num_pages, page_size, page_shift, num_kv_heads, head_dim;
};

struct WriteArgs {
  PoolArgs pool;
  void* k;  // writable aliases of pool.k / pool.v / scales
  void* v;
  float* k_scale;
  float* v_scale;
  const float* k_new;
  const float* v_new;
  const int32_t* slots;
  int64_t n_tokens;
};

struct GatherArgs {
  PoolArgs pool;
  const int32_t* table;
  int length;
  void* k_out;
  void* v_out;
  float* k_scale_out;
  float* v_scale_out;
};

// SLOT_MAPPING (block tables) and WINDOW_SLOT_MAPPING (rings)
struct SlotMapArgs {
  const int32_t* tables;     // [batch][width]
  const int32_t* positions;  // [batch][tokens]
  int32_t* slots;            // [batch][tokens]
  int batch, tokens, width, ring, page_shift, num_pages;
};

struct DecodeArgs {
  PoolArgs pool;
  const float* q;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;
  float* ws_acc;   // [batch][num_q_heads][n_split][head_dim], split index from the row's first
  float* ws_ml;    // [batch][num_q_heads][n_split][2]
  int* ws_ctrl;    // [4]: the item counter, the finished-workgroup counter (zero between calls)
  int* ws_arrive;  // [DECODE_ARRIVE_SLOTS]: splits stored per (sequence, head group) (zero between calls)
  int fuse_merge;  // 1: the last split of a (sequence, head group) merges; 0: a merge kernel follows
  int num_q_heads, group, max_blocks, batch, window, split_keys, n_split;
  int ring;        // 0: block j of a sequence is block_tables entry j; R > 0: entry j % R
  float qscale;    // scale * log2(e): scores come out in log2 units
};

// Decode workspace: 16 bytes of control words, then the arrival counters of the
// in-place merge (a fixed count, so no later call's counters overlap an earlier
// call's partial states), then the partial states.
constexpr int DECODE_BATCH_CHUNK = 2048;  // sequences per launch
constexpr int DECODE_ARRIVE_GROUPS = 64;  // head groups per sequence the counters cover
constexpr int64_t DECODE_ARRIVE_SLOTS = (int64_t)DECODE_BATCH_CHUNK * DECODE_ARRIVE_GROUPS;
constexpr int64_t DECODE_WS_HEADER = 16 + DECODE_ARRIVE_SLOTS * 4;

struct PrefillArgs {
  PoolArgs pool;
  const float* q;
  const int32_t* block_tables;
  const int32_t* positions;
  float* out;
  int num_q_heads, group, max_blocks, batch, tokens_per_row, window, n_qtiles, tokens_per_wg;
  int ring;        // 0: block j of a sequence is block_tables entry j; R > 0: entry j % R
  float qscale;
};

// Gated DeltaNet decode step over a slot-indexed state pool
struct GdnArgs {
  float* pool;          // [num_slots][num_heads][128][128] f32, updated in place
  const float *q, *k, *v, *g, *beta;  // [B][H][128] x3, [B][H] x2
  const int32_t* slots;      // [B], -1 = pad
  const int32_t* positions;  // [B], 0 = start from zero state
  float* out;                // [B][H][128]
  int batch, num_heads, num_slots;
};

// ------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are already validated.
hipError_t launch_write(const WriteArgs& a, int kv_dtype, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, int kv_dtype, hipStream_t s);
hipError_t launch_slot_mapping(const SlotMapArgs& a, hipStream_t s);
int decode_split_keys(int kv_dtype, int group, int head_dim, int page_size);
hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t s);
int prefill_tokens_per_wg(int group);
hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, hipStream_t s);
hipError_t launch_gdn_decode(const GdnArgs& a, hipStream_t s);
struct CopyPagesArgs {
  void *k, *v;
  float *k_scale, *v_scale;  // NULL for unscaled pools
  int num_pages;
  int64_t units;   // 16-byte units of K (and of V) per page
  int64_t scales;  // scales per page (num_kv_heads * page_size)
};
hipError_t launch_copy_pages(const CopyPagesArgs& p, const int32_t* src, const int32_t* dst, int n, hipStream_t s);
int set_error(int code, const char* msg);  // the thread's tl_last_error() text; returns code

}  // namespace tl
