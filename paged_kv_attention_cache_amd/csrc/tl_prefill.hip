// PAGED_ATTENTION, prefill entry: right-aligned rows, causal length = position + 1,
// optional sliding window, online softmax over key blocks ("How serving works in
// Tlaloc", section 1 prefill entries; section 2 PAGED_ATTENTION and blockwise
// bullets; section 3 sliding windows and chunked prefill).
//
// Design (gfx950):
// - One workgroup of 4 waves per (sequence b, kv head h, query tile).  A wave owns 32
//   query columns = (32/G tokens) x (G query heads of kv head h); the workgroup owns
//   128/G consecutive tokens of the row.  The sequence's pages are read once per
//   query tile (never per token) and shared through LDS by the 4 waves.
// - Keys are visited in tiles of 32 from the first key any of the tile's tokens can
//   see to the last position among them -- the pages' "first visible block .. block
//   of the last position" loop, taken at 32-key granularity; tiles a wave cannot see
//   are skipped by that wave.
// - Both dots are v_mfma_f32_32x32x2f32 (f32 operands, products and sums):
//     S^T[key, col] = sum_d K[key, d] Q[col, d]        (64 MFMAs per tile, D = 128)
//     O^T[d, col]  += sum_key V[key, d] P^T[key, col]  (64 MFMAs per tile)
//   The S^T accumulator of lane l holds 16 keys of column l % 32; the value product
//   needs, as its B operand, exactly those (key, column) pairs in the same
//   registers, provided its K-step s pairs the keys 8(s/4) + 4k + s%4 (k = lane half).
//   So probabilities stay in registers, and each lane's running max, sum and
//   rescale belong to its own column.  The d index is permuted in the score product
//   (lane half k covers d in [kD/2, (k+1)D/2)), which only reorders the f32 sum.
// - K/V tiles are widened to f32 in LDS (rows padded to D + 4 floats), double
//   buffered; the next tile's global loads are issued before the current tile's
//   MFMAs.
#include "tl_internal.h"

namespace tl {
namespace {

constexpr int NW = 4;        // waves per workgroup
constexpr int KT = 32;       // keys per tile
constexpr int COLS = 32;     // query columns per wave

template <int KVT, int D>
struct PrefillCfg {
  using Tr = KvTraits<KVT>;
  static constexpr int X = Tr::X;
  static constexpr int NC = D / X;                   // 16-byte units per K/V row
  static constexpr int UNITS = KT * NC;              // units per K (or V) tile
  static constexpr int UPT = (UNITS + NW * 64 - 1) / (NW * 64);  // units per thread
  static constexpr int LDR = D + 4;                  // LDS row stride (floats)
  static constexpr int TILE_FLOATS = KT * LDR;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// table entry of a sequence's block: the block itself, or its ring page's entry
__device__ __forceinline__ int ring_entry(const PrefillArgs& a, int blk) { return a.ring > 0 ? blk % a.ring : blk; }

template <int KVT, int D>
struct Staged {
  uint4 k[PrefillCfg<KVT, D>::UPT];
  uint4 v[PrefillCfg<KVT, D>::UPT];
  float ks[PrefillCfg<KVT, D>::UPT];
  float vs[PrefillCfg<KVT, D>::UPT];
};

// Keys are clamped into [key_lo, key_hi], the range some token of the workgroup can
// see: a tile's keys outside it (before a window's first key, past the last position)
// would read rows the caller never had to write, and although their probability is
// exactly 0, 0 times a non-finite stored value is NaN in the value product.  A clamped
// key re-reads a row inside the range, which is written and finite.
template <int KVT, int D>
__device__ __forceinline__ void stage_load(Staged<KVT, D>& st, const PrefillArgs& a, const int32_t* table,
                                           int h, int kt0, int key_lo, int key_hi, int tid) {
  using C = PrefillCfg<KVT, D>;
  const int S = a.pool.page_size, sh = a.pool.page_shift, H = a.pool.num_kv_heads;
#pragma unroll
  for (int i = 0; i < C::UPT; ++i) {
    const int u = tid + i * NW * 64;
    if (u < C::UNITS) {
      // K unit u: key u % KT, chunk u / KT  (chunked K layout: keys of a chunk contiguous)
      {
        const int kk = u % KT, c = u / KT;
        const int key = clampi(kt0 + kk, key_lo, key_hi);
        const int page = clampi(table[ring_entry(a, key >> sh)], 0, a.pool.num_pages - 1);
        const uint4* p = reinterpret_cast<const uint4*>(a.pool.k);
        st.k[i] = p[(((int64_t)page * H + h) * C::NC + c) * S + (key & (S - 1))];
        if constexpr (kv_scaled(KVT)) st.ks[i] = a.pool.k_scale[((int64_t)page * H + h) * S + (key & (S - 1))];
      }
      // V unit u: key u / NC, part u % NC (row-major V)
      {
        const int kk = u / C::NC, c = u % C::NC;
        const int key = clampi(kt0 + kk, key_lo, key_hi);
        const int page = clampi(table[ring_entry(a, key >> sh)], 0, a.pool.num_pages - 1);
        const uint4* p = reinterpret_cast<const uint4*>(a.pool.v);
        st.v[i] = p[(((int64_t)page * H + h) * S + (key & (S - 1))) * C::NC + c];
        if constexpr (kv_scaled(KVT)) st.vs[i] = a.pool.v_scale[((int64_t)page * H + h) * S + (key & (S - 1))];
      }
    }
  }
}

template <int KVT, int D>
__device__ __forceinline__ void stage_store(const Staged<KVT, D>& st, float* kl, float* vl, int tid) {
  using C = PrefillCfg<KVT, D>;
  constexpr int X = C::X;
#pragma unroll
  for (int i = 0; i < C::UPT; ++i) {
    const int u = tid + i * NW * 64;
    if (u < C::UNITS) {
      float x[X];
      {
        const int kk = u % KT, c = u / KT;
        widen_chunk<KVT>(st.k[i], x);
        if constexpr (kv_scaled(KVT)) {
#pragma unroll
          for (int e = 0; e < X; ++e) x[e] *= st.ks[i];
        }
        float* dst = kl + kk * C::LDR + c * X;
#pragma unroll
        for (int e = 0; e < X; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
      }
      {
        const int kk = u / C::NC, c = u % C::NC;
        widen_chunk<KVT>(st.v[i], x);
        if constexpr (kv_scaled(KVT)) {
#pragma unroll
          for (int e = 0; e < X; ++e) x[e] *= st.vs[i];
        }
        float* dst = vl + kk * C::LDR + c * X;
#pragma unroll
        for (int e = 0; e < X; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
      }
    }
  }
}

template <int KVT, int D, int G>
__global__ __launch_bounds__(NW * 64, 2) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<KVT, D>;
  constexpr int TPW = COLS / G;          // tokens per wave
  constexpr int TPG = TPW * NW;          // tokens per workgroup
  constexpr int HALF = D / 2;
  constexpr int NDB = D / 32;            // 32-row blocks of d in O^T
  __shared__ float lds[2][2][C::TILE_FLOATS];  // [buffer][K|V][key][d]
  __shared__ int red[2][NW];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  // Work order: query tiles latest-first across all rows and heads (rows are
  // right-aligned, so a later tile holds later positions and sees more keys).  The
  // dispatcher hands out launch ids in order, round-robin over the XCDs, so the heavy
  // tiles of every row start first and spread over the whole chip; the light ones
  // (and the pad-only tiles, which return at once) fill the end.  Within a tile step
  // the rows rotate from one step to the next: the hand-out below the XCD level also
  // follows the launch id, and without the rotation each of its partitions would get
  // the same rows at every step, so the one holding the longest rows would set the time.
  const int nx = gridDim.x, ny = gridDim.y, nz = gridDim.z;
  const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int step = lin / (ny * nz);
  const int tile = nx - 1 - step;
  const int h = lin % ny;
  const int b = (lin / ny + step) % nz;

  const int T = a.tokens_per_row;
  const int tok = tile * TPG + w * TPW + col / G;
  const int g = col % G;
  const int hq = h * G + g;
  const int max_pos = a.ring > 0 ? 0x7FFFFFFF : a.max_blocks * a.pool.page_size - 1;  // a ring has no end
  int pos = -1;
  if (tok < T) pos = min(a.positions[(int64_t)b * T + tok], max_pos);
  const int plo = (pos < 0) ? 0 : (a.window > 0 ? max(0, pos - a.window + 1) : 0);
  const bool live = pos >= 0;

  // workgroup key range [klo, khi] and this wave's own range
  int wlo = live ? plo : 0x7FFFFFFF, whi = live ? pos : -1;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) { wlo = min(wlo, __shfl_xor(wlo, m, 64)); whi = max(whi, __shfl_xor(whi, m, 64)); }
  if (lane == 0) { red[0][w] = wlo; red[1][w] = whi; }
  __syncthreads();
  int klo = red[0][0], khi = red[1][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) { klo = min(klo, red[0][i]); khi = max(khi, red[1][i]); }
  const int w_lo = wlo, w_hi = whi;

  float* orow = a.out + (((int64_t)b * T + tok) * a.num_q_heads + hq) * D;
  if (khi < 0) {  // no live token in this tile: all-zero outputs
    if (tok < T) {
#pragma unroll
      for (int d = half * HALF; d < (half + 1) * HALF; d += 4) *reinterpret_cast<float4*>(orow + d) = make_float4(0, 0, 0, 0);
    }
    return;
  }
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;

  // queries: this lane's column, d in [half*D/2, (half+1)*D/2), pre-scaled
  float q[HALF];
  {
    const float* qp = a.q + (((int64_t)b * T + min(tok, T - 1)) * a.num_q_heads + hq) * D + half * HALF;
#pragma unroll
    for (int d = 0; d < HALF; d += 4) {
      float4 x = live ? *reinterpret_cast<const float4*>(qp + d) : make_float4(0, 0, 0, 0);
      q[d] = x.x * a.qscale; q[d + 1] = x.y * a.qscale; q[d + 2] = x.z * a.qscale; q[d + 3] = x.w * a.qscale;
    }
  }

  v16f o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = v16f{};
  float m = -INFINITY, l = 0.0f;

  const int t_first = klo / KT, t_last = khi / KT;
  Staged<KVT, D> st;
  stage_load<KVT, D>(st, a, table, h, t_first * KT, klo, khi, tid);
  stage_store<KVT, D>(st, lds[0][0], lds[0][1], tid);
  __syncthreads();

  for (int t = t_first; t <= t_last; ++t) {
    const int buf = (t - t_first) & 1;
    const bool more = t < t_last;
    if (more) stage_load<KVT, D>(st, a, table, h, (t + 1) * KT, klo, khi, tid);
    const int kt0 = t * KT;
    if (kt0 <= w_hi && kt0 + KT - 1 >= w_lo) {
      const float* kl = lds[buf][0];
      const float* vl = lds[buf][1];
      // ---- S^T = K Q^T
      v16f s = v16f{};
      const float* krow = kl + col * C::LDR + half * HALF;
#pragma unroll
      for (int d = 0; d < HALF; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + d);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, q[d], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, q[d + 1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, q[d + 2], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, q[d + 3], s, 0, 0, 0);
      }
      // ---- mask and online softmax for this lane's column
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt0 + 8 * (r / 4) + 4 * half + (r % 4);
        const bool vis = live && key >= plo && key <= pos;
        s[r] = vis ? s[r] : -INFINITY;
        tmax = fmaxf(tmax, s[r]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = fast_exp2(s[r] - m_use); psum += s[r]; }
      l = l * alpha + psum;
      m = m_new;
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[i] *= alpha;
      // ---- O^T += V^T P^T, K-step r pairs keys 8(r/4) + 4*half + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r / 4) + 4 * half + (r % 4);
        const float* vrow = vl + kk * C::LDR + col;
#pragma unroll
        for (int i = 0; i < NDB; ++i) o[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[i * 32], s[r], o[i], 0, 0, 0);
      }
    }
    if (more) stage_store<KVT, D>(st, lds[buf ^ 1][0], lds[buf ^ 1][1], tid);
    __syncthreads();
  }

  // ---- normalise and write: o[i] register r holds d = 32i + 8(r/4) + 4*half + r%4
  l += __shfl_xor(l, 32, 64);
  if (tok < T) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * i + 8 * r4 + 4 * half;
        float4 v = l > 0.0f ? make_float4(o[i][4 * r4] * inv, o[i][4 * r4 + 1] * inv, o[i][4 * r4 + 2] * inv,
                                          o[i][4 * r4 + 3] * inv)
                            : make_float4(0, 0, 0, 0);
        *reinterpret_cast<float4*>(orow + d) = v;
      }
    }
  }
}

template <int KVT, int D>
hipError_t prefill_dispatch_d(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid(a.n_qtiles, a.pool.num_kv_heads, a.batch);
  switch (a.group) {
    case 8: hipLaunchKernelGGL((prefill_kernel<KVT, D, 8>), grid, dim3(NW * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<KVT, D, 4>), grid, dim3(NW * 64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<KVT, D, 2>), grid, dim3(NW * 64), 0, s, a); break;
    default: hipLaunchKernelGGL((prefill_kernel<KVT, D, 1>), grid, dim3(NW * 64), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int KVT>
hipError_t prefill_dispatch(const PrefillArgs& a, hipStream_t s) {
  if (a.pool.head_dim == 128) return prefill_dispatch_d<KVT, 128>(a, s);
  return prefill_dispatch_d<KVT, 64>(a, s);
}

}  // namespace

int prefill_tokens_per_wg(int group) { return NW * COLS / group; }

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, hipStream_t s) {
  if (a.batch == 0 || a.tokens_per_row == 0) return hipSuccess;
  switch (kv_dtype) {
    case KV_F32: return prefill_dispatch<KV_F32>(a, s);
    case KV_BF16: return prefill_dispatch<KV_BF16>(a, s);
    case KV_FP8: return prefill_dispatch<KV_FP8>(a, s);
    case KV_FP8U: return prefill_dispatch<KV_FP8U>(a, s);
    default: return prefill_dispatch<KV_INT8>(a, s);
  }
}

}  // namespace tl
