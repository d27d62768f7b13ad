// KV_CACHE_WRITE: scatter new K/V rows into the page pool at their slots
// ("How serving works in Tlaloc", section 2, KV_CACHE_WRITE bullet; slot -1 is a pad
// whose KV is never written, section 1), the slot mapping that names those slots
// (section 3: SLOT_MAPPING, and WINDOW_SLOT_MAPPING for a ring), and the test gather
// that copies a sequence's stored rows out in logical order.
//
// Mapping: 8 lanes own one (token, kv head) row of D values; the 8 rows of a wave
// are 8 consecutive tokens of one head, and each lane holds whole 16-byte store
// units of the encoded row, interleaved across the 8 lanes, so every store
// instruction writes whole lines of the K and V pages when slots are consecutive.
// The stored encodings are those of include/tl.h.  HBM-bound: each row is read
// once in f32 and written once in the pool dtype.
#include "tl_internal.h"

namespace tl {
namespace {

constexpr int ROW_LANES = 8;
constexpr int WG = 256;
typedef unsigned int wu4 __attribute__((ext_vector_type(4)));
typedef unsigned int wu2 __attribute__((ext_vector_type(2)));

// Every byte is read or written once.  Measured on a 62.5K-token bf16 history chunk
// and a 52K-token fp8 one: f32/bf16 pools stream best with nontemporal loads and
// plain stores, fp8 pools (a quarter of the bytes written, more arithmetic per byte)
// with plain loads and nontemporal stores.
template <bool NT, typename V>
__device__ __forceinline__ void wst(V x, V* p) {
  if constexpr (NT) __builtin_nontemporal_store(x, p); else *p = x;
}
template <bool NT>
__device__ __forceinline__ wu4 wld(const wu4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p); else return *p;
}

template <int KVT, int D>
__device__ __forceinline__ void encode_row(const float (&x)[D / ROW_LANES], typename KvTraits<KVT>::T (&enc)[D / ROW_LANES],
                                           float& scale) {
  using Tr = KvTraits<KVT>;
  constexpr int E = D / ROW_LANES;
  scale = 1.0f;
  if constexpr (KVT == KV_F32) {
#pragma unroll
    for (int i = 0; i < E; ++i) enc[i] = x[i];
  } else if constexpr (KVT == KV_BF16) {
#pragma unroll
    for (int i = 0; i < E; ++i) enc[i] = (uint16_t)f32_to_bf16(x[i]);
  } else if constexpr (KVT == KV_INT8) {
    // the int8 formula per row: scale = absmax / 127 (1 for a zero row), codes rounded
    // half to even and clamped to +-127, both divisions IEEE f32
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(x[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    scale = (m == 0.0f) ? 1.0f : m / 127.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float y = fminf(fmaxf(__builtin_rintf(x[i] / scale), -127.0f), 127.0f);
      enc[i] = (uint8_t)(int8_t)(int)y;
    }
  } else if constexpr (KVT == KV_FP8U) {
    // no scale: the value itself, saturated at +-448, to the nearest code
#pragma unroll
    for (int i = 0; i < E; i += 2) {
      const float y0 = fminf(fmaxf(x[i], -448.0f), 448.0f);
      const float y1 = fminf(fmaxf(x[i + 1], -448.0f), 448.0f);
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      enc[i] = (uint8_t)(w & 0xFF);
      enc[i + 1] = (uint8_t)((w >> 8) & 0xFF);
    }
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(x[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    scale = (m == 0.0f) ? 1.0f : m / 448.0f;  // IEEE f32 divide
#pragma unroll
    for (int i = 0; i < E; i += 2) {
      float y0 = fminf(fmaxf(x[i] / scale, -448.0f), 448.0f);
      float y1 = fminf(fmaxf(x[i + 1] / scale, -448.0f), 448.0f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      enc[i] = (uint8_t)(w & 0xFF);
      enc[i + 1] = (uint8_t)((w >> 8) & 0xFF);
    }
  }
  (void)sizeof(Tr);
}

// Rows are (token, kv head) pairs, ordered so that the 8 rows of a wave's lane group
// are 8 consecutive tokens of one head: their K chunks and V rows then land next to
// each other in the pool when their slots are consecutive (history writes).  Every
// byte is read or written once, so loads and stores are nontemporal.
template <int KVT, int D>
__global__ __launch_bounds__(WG) void write_kernel(WriteArgs a) {
  using Tr = KvTraits<KVT>;
  typedef typename Tr::T T;
  typedef wu4 u4;
  typedef wu2 u2;
  constexpr int E = D / ROW_LANES;   // values per lane
  constexpr int X = Tr::X;           // values per 16-byte chunk
  constexpr int NC = D / X;          // chunks per row
  const int lane_in_row = threadIdx.x % ROW_LANES;
  const int64_t r = (int64_t)blockIdx.x * (WG / ROW_LANES) + threadIdx.x / ROW_LANES;
  const int H = a.pool.num_kv_heads;
  // r -> (token block of 8, head, token in block)
  const int64_t blk = r / (8 * H);
  const int h = (int)((r / 8) % H);
  const int64_t token = blk * 8 + (r % 8);
  if (token >= a.n_tokens) return;
  const int32_t slot = a.slots[token];
  const int64_t limit = (int64_t)a.pool.num_pages * a.pool.page_size;
  if (slot < 0 || slot >= limit) return;  // -1 is a pad; anything else out of range is skipped
  const int S = a.pool.page_size;
  const int page = slot >> a.pool.page_shift;
  const int off = slot & (S - 1);
  const int64_t row = token * H + h;
  // A unit is UE consecutive values whose encoding is one store (16 bytes, or 8 for
  // fp8 rows of 64); lane j of the row's 8 owns units j, j + 8, ... so that each store
  // instruction of the 8 lanes covers one contiguous span of the destination.
  constexpr int UE = (X * ROW_LANES <= D) ? X : D / ROW_LANES;
  constexpr int NU = E / UE;  // units per lane
  constexpr bool NTL = Tr::BYTES != 1, NTS = Tr::BYTES == 1;
  float xk[E], xv[E];
  {
    const u4* sk = reinterpret_cast<const u4*>(a.k_new + row * D);
    const u4* sv = reinterpret_cast<const u4*>(a.v_new + row * D);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
#pragma unroll
      for (int q = 0; q < UE / 4; ++q) {
        const int at = (UE * (lane_in_row + ROW_LANES * i)) / 4 + q;
        const u4 tk = wld<NTL>(sk + at);
        const u4 tv = wld<NTL>(sv + at);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xk[i * UE + 4 * q + e] = __uint_as_float(tk[e]);
          xv[i * UE + 4 * q + e] = __uint_as_float(tv[e]);
        }
      }
    }
  }
  T ek[E], ev[E];
  float sck, scv;
  encode_row<KVT, D>(xk, ek, sck);
  encode_row<KVT, D>(xv, ev, scv);
  constexpr int W = UE * Tr::BYTES;
  static_assert(W == 16 || W == 8, "unit is one 16- or 8-byte store");
  {
    T* kb = reinterpret_cast<T*>(a.k);
    T* vrow = reinterpret_cast<T*>(a.v) + (((int64_t)page * H + h) * S + off) * D;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int d = UE * (lane_in_row + ROW_LANES * i);
      const int c = d / X, e = d % X;
      T* kd = kb + ((((int64_t)page * H + h) * NC + c) * S + off) * X + e;
      if constexpr (W == 16) {
        wst<NTS>(*reinterpret_cast<const u4*>(&ek[i * UE]), reinterpret_cast<u4*>(kd));
        wst<NTS>(*reinterpret_cast<const u4*>(&ev[i * UE]), reinterpret_cast<u4*>(vrow + d));
      } else {
        wst<NTS>(*reinterpret_cast<const u2*>(&ek[i * UE]), reinterpret_cast<u2*>(kd));
        wst<NTS>(*reinterpret_cast<const u2*>(&ev[i * UE]), reinterpret_cast<u2*>(vrow + d));
      }
    }
  }
  if constexpr (kv_scaled(KVT)) {
    if (lane_in_row == 0) {
      const int64_t si = ((int64_t)page * H + h) * S + off;
      a.k_scale[si] = sck;
      a.v_scale[si] = scv;
    }
  }
}

// One thread per 16-byte unit of the logical output [length][H][D] (and per scale).
template <int KVT, int D>
__global__ __launch_bounds__(WG) void gather_kernel(GatherArgs a) {
  using Tr = KvTraits<KVT>;
  constexpr int X = Tr::X;
  constexpr int NC = D / X;  // 16-byte units per row
  const int H = a.pool.num_kv_heads, S = a.pool.page_size;
  const int64_t units = (int64_t)a.length * H * NC;
  const int64_t u = (int64_t)blockIdx.x * WG + threadIdx.x;
  if (u < units) {
    const int c = (int)(u % NC);
    const int64_t r = u / NC;
    const int h = (int)(r % H);
    const int j = (int)(r / H);
    int page = a.table[j >> a.pool.page_shift];
    page = min(max(page, 0), a.pool.num_pages - 1);
    const int off = j & (S - 1);
    const uint4* ks = reinterpret_cast<const uint4*>(a.pool.k);
    const uint4* vs = reinterpret_cast<const uint4*>(a.pool.v);
    uint4 kv = ks[(((int64_t)page * H + h) * NC + c) * S + off];
    uint4 vv = vs[(((int64_t)page * H + h) * S + off) * NC + c];
    reinterpret_cast<uint4*>(a.k_out)[u] = kv;
    reinterpret_cast<uint4*>(a.v_out)[u] = vv;
  }
  if constexpr (kv_scaled(KVT)) {
    const int64_t n = (int64_t)a.length * H;
    if (u < n) {
      const int h = (int)(u % H);
      const int j = (int)(u / H);
      int page = a.table[j >> a.pool.page_shift];
      page = min(max(page, 0), a.pool.num_pages - 1);
      const int64_t idx = ((int64_t)page * H + h) * S + (j & (S - 1));
      a.k_scale_out[u] = a.pool.k_scale[idx];
      a.v_scale_out[u] = a.pool.v_scale[idx];
    }
  }
}

// Slot of each (row, token): the block's table entry times the page size plus the
// offset in the page; on a ring, block j is on entry j % R.  A pad (position < 0), a
// block past the table and an entry outside the pool all give -1, which the write
// skips.  One thread per token.
__global__ __launch_bounds__(WG) void slot_mapping_kernel(SlotMapArgs a) {
  const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
  if (i >= (int64_t)a.batch * a.tokens) return;
  const int64_t b = i / a.tokens;
  const int p = a.positions[i];
  int32_t slot = -1;
  if (p >= 0) {
    int blk = p >> a.page_shift;
    if (a.ring > 0) blk %= a.ring;
    if (blk < a.width) {
      const int page = a.tables[b * a.width + blk];
      if (page >= 0 && page < a.num_pages) slot = (page << a.page_shift) | (p & ((1 << a.page_shift) - 1));
    }
  }
  a.slots[i] = slot;
}

template <int KVT>
hipError_t write_dispatch(const WriteArgs& a, hipStream_t s) {
  // rows are counted in whole blocks of 8 tokens (the tail block's missing tokens return)
  const int64_t rows = ((a.n_tokens + 7) / 8) * 8 * a.pool.num_kv_heads;
  const dim3 grid((unsigned)((rows + (WG / ROW_LANES) - 1) / (WG / ROW_LANES)));
  if (a.pool.head_dim == 128) hipLaunchKernelGGL((write_kernel<KVT, 128>), grid, dim3(WG), 0, s, a);
  else hipLaunchKernelGGL((write_kernel<KVT, 64>), grid, dim3(WG), 0, s, a);
  return hipGetLastError();
}

template <int KVT>
hipError_t gather_dispatch(const GatherArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.length * a.pool.num_kv_heads * (a.pool.head_dim / KvTraits<KVT>::X);
  const dim3 grid((unsigned)((units + WG - 1) / WG));
  if (a.pool.head_dim == 128) hipLaunchKernelGGL((gather_kernel<KVT, 128>), grid, dim3(WG), 0, s, a);
  else hipLaunchKernelGGL((gather_kernel<KVT, 64>), grid, dim3(WG), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, int kv_dtype, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  switch (kv_dtype) {
    case KV_F32: return write_dispatch<KV_F32>(a, s);
    case KV_BF16: return write_dispatch<KV_BF16>(a, s);
    case KV_FP8: return write_dispatch<KV_FP8>(a, s);
    case KV_FP8U: return write_dispatch<KV_FP8U>(a, s);
    default: return write_dispatch<KV_INT8>(a, s);
  }
}

hipError_t launch_slot_mapping(const SlotMapArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.batch * a.tokens;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)((n + WG - 1) / WG)), dim3(WG), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, int kv_dtype, hipStream_t s) {
  if (a.length == 0) return hipSuccess;
  switch (kv_dtype) {
    case KV_F32: return gather_dispatch<KV_F32>(a, s);
    case KV_BF16: return gather_dispatch<KV_BF16>(a, s);
    case KV_FP8: return gather_dispatch<KV_FP8>(a, s);
    case KV_FP8U: return gather_dispatch<KV_FP8U>(a, s);
    default: return gather_dispatch<KV_INT8>(a, s);
  }
}

}  // namespace tl
