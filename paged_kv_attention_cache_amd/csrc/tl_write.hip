// KV_CACHE_WRITE: scatter new K/V rows into the page pool at their slots
// ("How serving works in Tlaloc", section 2, KV_CACHE_WRITE bullet; slot -1 is a pad
// whose KV is never written, section 1).  Also the test gather that copies a
// sequence's stored rows out in logical order.
//
// Mapping: 8 lanes own one (token, kv head) row of D values, each lane D/8
// contiguous values, so a wave reads 8 consecutive rows = one contiguous span of
// k_new.  The stored encodings are those of include/tl.h.  HBM-bound: each row is
// read once in f32 and written once in the pool dtype.
#include "tl_internal.h"

namespace tl {
namespace {

constexpr int ROW_LANES = 8;
constexpr int WG = 256;

template <int KVT, int D>
__global__ __launch_bounds__(WG) void write_kernel(WriteArgs a) {
  using Tr = KvTraits<KVT>;
  constexpr int E = D / ROW_LANES;   // values per lane
  constexpr int X = Tr::X;           // values per 16-byte chunk
  constexpr int NC = D / X;          // chunks per row
  const int lane_in_row = threadIdx.x % ROW_LANES;
  const int64_t row = (int64_t)blockIdx.x * (WG / ROW_LANES) + threadIdx.x / ROW_LANES;
  const int H = a.pool.num_kv_heads;
  const int64_t rows = a.n_tokens * H;
  if (row >= rows) return;
  const int64_t token = row / H;
  const int h = (int)(row - token * H);
  const int32_t slot = a.slots[token];
  const int64_t limit = (int64_t)a.pool.num_pages * a.pool.page_size;
  if (slot < 0 || slot >= limit) return;  // -1 is a pad; anything else out of range is skipped
  const int S = a.pool.page_size;
  const int page = slot >> a.pool.page_shift;
  const int off = slot & (S - 1);
  const int d0 = lane_in_row * E;

  for (int which = 0; which < 2; ++which) {
    const float* src = (which == 0 ? a.k_new : a.v_new) + row * D + d0;
    float x[E];
#pragma unroll
    for (int i = 0; i < E; i += 4) {
      float4 t = *reinterpret_cast<const float4*>(src + i);
      x[i] = t.x; x[i + 1] = t.y; x[i + 2] = t.z; x[i + 3] = t.w;
    }
    typename Tr::T enc[E];
    float scale = 1.0f;
    if constexpr (KVT == KV_F32) {
#pragma unroll
      for (int i = 0; i < E; ++i) enc[i] = x[i];
    } else if constexpr (KVT == KV_BF16) {
#pragma unroll
      for (int i = 0; i < E; ++i) enc[i] = (uint16_t)f32_to_bf16(x[i]);
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
    typename Tr::T* base = reinterpret_cast<typename Tr::T*>(which == 0 ? a.k : a.v);
    if (which == 0) {
      // K: [page][h][D/X][S][X]; this lane's E values cover whole or half chunks
#pragma unroll
      for (int i = 0; i < E; i += (E < X ? E : X)) {
        const int d = d0 + i;
        const int c = d / X, e = d % X;
        typename Tr::T* dst = base + ((((int64_t)page * H + h) * NC + c) * S + off) * X + e;
        constexpr int W = (E < X ? E : X) * Tr::BYTES;
        if constexpr (W == 16) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&enc[i]);
        } else {
          *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(&enc[i]);
        }
      }
    } else {
      // V: [page][h][S][D], contiguous row
      typename Tr::T* dst = base + (((int64_t)page * H + h) * S + off) * D + d0;
      constexpr int BYTES = E * Tr::BYTES;
#pragma unroll
      for (int i = 0; i < BYTES / 16; ++i)
        reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(enc)[i];
      if constexpr (BYTES % 16 == 8) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(enc);
    }
    if constexpr (KVT == KV_FP8) {
      if (lane_in_row == 0) {
        float* sc = (which == 0 ? a.k_scale : a.v_scale);
        sc[((int64_t)page * H + h) * S + off] = scale;
      }
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
  if constexpr (KVT == KV_FP8) {
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

template <int KVT>
hipError_t write_dispatch(const WriteArgs& a, hipStream_t s) {
  const int64_t rows = a.n_tokens * a.pool.num_kv_heads;
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
    default: return write_dispatch<KV_FP8>(a, s);
  }
}

hipError_t launch_gather(const GatherArgs& a, int kv_dtype, hipStream_t s) {
  if (a.length == 0) return hipSuccess;
  switch (kv_dtype) {
    case KV_F32: return gather_dispatch<KV_F32>(a, s);
    case KV_BF16: return gather_dispatch<KV_BF16>(a, s);
    default: return gather_dispatch<KV_FP8>(a, s);
  }
}

}  // namespace tl
