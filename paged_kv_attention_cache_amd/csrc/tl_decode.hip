// PAGED_ATTENTION, decode entry: one new token per sequence attends over the pages
// its block table names ("How serving works in Tlaloc", section 2, PAGED_ATTENTION
// bullet: gather the pages, f32 dots, masked softmax; section 3: sliding window).
//
// Design (gfx950):
// - Split-K.  The context of a sequence is cut into splits of a fixed number of keys
//   (chosen from the pool geometry only), so a sequence's partition depends on its
//   own length alone.  One wave per (sequence, head slot pair, split) computes the
//   split's softmax state (m, l, acc); a merge kernel combines the splits of
//   sequences that have more than one.
// - Both dots run on the matrix cores as v_mfma_f32_4x4x1f32 (16 blocks of 4x4x1,
//   f32 operands, products and sums).  A wave holds two "slots" of 4 query heads
//   each (lanes 0-31 and 32-63): two head groups of one KV head when G = 8, or two
//   KV heads when G <= 4.  A tile is 32 keys per slot.
//     scores   S[key, head] += K[key, d] * Q[head, d]   one MFMA per d; lane = key
//     values   O[head, d]   += P[head, key] * V[key, d] one MFMA per key and 32 d
//   The score accumulator of lane (slot, key group kg, head j) holds keys kg*4+r in
//   register r, which is exactly the A operand the value product needs, broadcast
//   from block kg to the slot's 8 blocks by the MFMA's CBSZ/ABID controls.  So the
//   probabilities never leave registers.
// - K pages are stored in 16-byte chunks key-major ([page][head][D/x][S][x]), so the
//   32 keys of a tile read one chunk each from one contiguous 512-byte span.  V rows
//   are read one key at a time by all lanes (one coalesced row per load).  The next
//   tile's K, V and scales are loaded into registers while the current one computes.
// - fp8: the per-(token, head) K scale multiplies the finished dot; the V scale
//   multiplies the probability before the value product (the sum over keys is
//   unchanged, since both are per key).
#include "tl_internal.h"

namespace tl {
namespace {

constexpr int TK = 32;  // keys per tile per slot

template <int KVT, int D>
struct Tile {
  using Tr = KvTraits<KVT>;
  static constexpr int NC = D / Tr::X;             // K chunks per key
  static constexpr int NT = D / 32;                // value MFMAs per key (d per lane)
  static constexpr int VW = NT * Tr::BYTES;        // bytes of V per lane per key
  static constexpr int VWORDS = (VW + 3) / 4;
  uint4 k[NC];
  uint32_t v[TK][VWORDS];
  v4f ks, vs;                                      // fp8 scales of keys kg*4 + r
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <int KVT, int D>
__device__ __forceinline__ void load_tile(Tile<KVT, D>& t, const DecodeArgs& a, const int32_t* table,
                                          int kvh, int k0, int lo, int hi, int lane) {
  using TL = Tile<KVT, D>;
  const int S = a.pool.page_size, sh = a.pool.page_shift, H = a.pool.num_kv_heads;
  const int kg = (lane >> 2) & 7, j = lane & 3;
  // K: this lane's key
  {
    const int key = clampi(k0 + kg * 4 + j, lo, hi);
    const int page = clampi(table[key >> sh], 0, a.pool.num_pages - 1);
    const uint4* base = reinterpret_cast<const uint4*>(a.pool.k) +
                        (((int64_t)page * H + kvh) * TL::NC) * S + (key & (S - 1));
#pragma unroll
    for (int c = 0; c < TL::NC; ++c) t.k[c] = base[(int64_t)c * S];
  }
  // fp8 scales of keys kg*4 .. kg*4+3 (one page: groups of 4 never straddle pages)
  if constexpr (KVT == KV_FP8) {
    const int g0 = clampi(k0 + kg * 4, lo & ~3, hi & ~3);
    const int page = clampi(table[g0 >> sh], 0, a.pool.num_pages - 1);
    const int64_t idx = ((int64_t)page * H + kvh) * S + (g0 & (S - 1));
    t.ks = *reinterpret_cast<const v4f*>(a.pool.k_scale + idx);
    t.vs = *reinterpret_cast<const v4f*>(a.pool.v_scale + idx);
  }
  // V: every lane reads NT values of each key's row
  const int d0 = (lane & 31) * TL::NT;
#pragma unroll
  for (int kk = 0; kk < TK; ++kk) {
    const int key = clampi(k0 + kk, lo, hi);
    const int page = clampi(table[key >> sh], 0, a.pool.num_pages - 1);
    const char* row = reinterpret_cast<const char*>(a.pool.v) +
                      ((((int64_t)page * H + kvh) * S + (key & (S - 1))) * D + d0) * KvTraits<KVT>::BYTES;
    if constexpr (TL::VW == 16) {
      uint4 x = *reinterpret_cast<const uint4*>(row);
      t.v[kk][0] = x.x; t.v[kk][1] = x.y; t.v[kk][2] = x.z; t.v[kk][3] = x.w;
    } else if constexpr (TL::VW == 8) {
      uint2 x = *reinterpret_cast<const uint2*>(row);
      t.v[kk][0] = x.x; t.v[kk][1] = x.y;
    } else if constexpr (TL::VW == 4) {
      t.v[kk][0] = *reinterpret_cast<const uint32_t*>(row);
    } else {  // fp8 with D = 64: 2 bytes
      t.v[kk][0] = *reinterpret_cast<const uint16_t*>(row);
    }
  }
}

// widen the NT value elements of key kk for this lane
template <int KVT, int D>
__device__ __forceinline__ void widen_v(const Tile<KVT, D>& t, int kk, float* o) {
  using TL = Tile<KVT, D>;
  if constexpr (KVT == KV_F32) {
#pragma unroll
    for (int i = 0; i < TL::NT; ++i) o[i] = __uint_as_float(t.v[kk][i]);
  } else if constexpr (KVT == KV_BF16) {
#pragma unroll
    for (int i = 0; i < TL::NT / 2; ++i) { o[2 * i] = bf16_lo(t.v[kk][i]); o[2 * i + 1] = bf16_hi(t.v[kk][i]); }
  } else {
    if constexpr (TL::NT == 4) {
      fp8x4_to_f32(t.v[kk][0], o);
    } else {
      typedef float v2f __attribute__((ext_vector_type(2)));
      v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)t.v[kk][0], false);
      o[0] = lo[0]; o[1] = lo[1];
    }
  }
}

// values: O[t] += P(key kg*4 + r) * V(key, d(lane, t)), with P broadcast from block KG
template <int KVT, int D, int KG>
__device__ __forceinline__ void pv_group(const Tile<KVT, D>& t, const float* pv, v4f* o) {
  using TL = Tile<KVT, D>;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float vv[TL::NT];
    widen_v<KVT, D>(t, KG * 4 + r, vv);
#pragma unroll
    for (int i = 0; i < TL::NT; ++i) o[i] = __builtin_amdgcn_mfma_f32_4x4x1f32(pv[r], vv[i], o[i], 3, KG, 0);
  }
}

template <int KVT, int D, int G>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using TL = Tile<KVT, D>;
  constexpr int X = KvTraits<KVT>::X;
  constexpr int NT = TL::NT;
  const int lane = threadIdx.x;
  const int slot = lane >> 5, kg = (lane >> 2) & 7, j = lane & 3;
  const int split = blockIdx.x, b = blockIdx.z;
  const int H = a.pool.num_kv_heads;
  // slot -> kv head and the q heads it holds
  int kvh, qh_base;
  bool slot_on;
  if constexpr (G == 8) {
    kvh = blockIdx.y; qh_base = kvh * 8 + slot * 4; slot_on = true;
  } else {
    kvh = blockIdx.y * 2 + slot; slot_on = kvh < H; qh_base = kvh * G;
    if (!slot_on) kvh = H - 1;  // keep addresses valid; results are discarded
  }
  const bool head_on = slot_on && (G >= 4 || j < G);

  const int L = min(a.seq_lens[b], a.max_blocks * a.pool.page_size);
  if (L <= 0) return;
  const int hi = L - 1;
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int s_first = lo / a.split_keys, s_last = hi / a.split_keys;
  if (split < s_first || split > s_last) return;
  const int k_begin = max(split * a.split_keys, lo) & ~(TK - 1);
  const int k_end = min((split + 1) * a.split_keys - 1, hi);  // inclusive
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;

  // queries of this lane's head, pre-scaled by scale * log2(e)
  float q[D];
  {
    const float* qp = a.q + ((int64_t)b * a.num_q_heads + qh_base + j) * D;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      float4 x = head_on ? *reinterpret_cast<const float4*>(qp + d) : make_float4(0, 0, 0, 0);
      q[d] = x.x * a.qscale; q[d + 1] = x.y * a.qscale; q[d + 2] = x.z * a.qscale; q[d + 3] = x.w * a.qscale;
    }
  }

  v4f o[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) o[i] = v4f{0, 0, 0, 0};
  float m = -INFINITY, l = 0.0f;

  TL cur, nxt;
  load_tile<KVT, D>(cur, a, table, kvh, k_begin, lo, hi, lane);
  for (int k0 = k_begin; k0 <= k_end; k0 += TK) {
    const bool more = k0 + TK <= k_end;
    if (more) load_tile<KVT, D>(nxt, a, table, kvh, k0 + TK, lo, hi, lane);

    // ---- scores: 4 independent accumulation chains over d
    v4f s4[4] = {v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}};
#pragma unroll
    for (int c = 0; c < TL::NC; ++c) {
      float kv[X];
      widen_chunk<KVT>(cur.k[c], kv);
#pragma unroll
      for (int e = 0; e < X; ++e)
        s4[e & 3] = __builtin_amdgcn_mfma_f32_4x4x1f32(kv[e], q[c * X + e], s4[e & 3], 0, 0, 0);
    }
    v4f sc = (s4[0] + s4[1]) + (s4[2] + s4[3]);

    // ---- mask, online softmax (per head = per lane j within the slot)
    float s[4], tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0 + kg * 4 + r;
      const bool valid = key >= lo && key <= k_end;
      float x = sc[r];
      if constexpr (KVT == KV_FP8) x *= cur.ks[r];
      s[r] = valid ? x : -INFINITY;
      tmax = fmaxf(tmax, s[r]);
    }
    tmax = wave_xor_max(tmax, 4);
    tmax = wave_xor_max(tmax, 8);
    tmax = wave_xor_max(tmax, 16);
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float p[4], psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(s[r] - m_use);
      psum += p[r];
    }
    l = l * alpha + psum;
    m = m_new;
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (KVT == KV_FP8) pv[r] = (s[r] == -INFINITY) ? 0.0f : p[r] * cur.vs[r];
      else pv[r] = p[r];
    }
    // rescale the value accumulators: register r of lane (quad) holds head r of the slot
    const float a0 = quad_bcast<0>(alpha), a1 = quad_bcast<1>(alpha);
    const float a2 = quad_bcast<2>(alpha), a3 = quad_bcast<3>(alpha);
#pragma unroll
    for (int i = 0; i < NT; ++i) { o[i][0] *= a0; o[i][1] *= a1; o[i][2] *= a2; o[i][3] *= a3; }

    // ---- values
    pv_group<KVT, D, 0>(cur, pv, o);
    pv_group<KVT, D, 1>(cur, pv, o);
    pv_group<KVT, D, 2>(cur, pv, o);
    pv_group<KVT, D, 3>(cur, pv, o);
    pv_group<KVT, D, 4>(cur, pv, o);
    pv_group<KVT, D, 5>(cur, pv, o);
    pv_group<KVT, D, 6>(cur, pv, o);
    pv_group<KVT, D, 7>(cur, pv, o);

    if (more) cur = nxt;
  }

  // ---- finish: l per head summed over the slot's key groups
  l = wave_xor_sum(l, 4);
  l = wave_xor_sum(l, 8);
  l = wave_xor_sum(l, 16);
  const float lr[4] = {quad_bcast<0>(l), quad_bcast<1>(l), quad_bcast<2>(l), quad_bcast<3>(l)};
  const int d0 = (lane & 31) * NT;
  const bool single = (s_first == s_last);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!slot_on || (G < 4 && r >= G)) continue;
    const int hq = qh_base + r;
    float vals[NT];
    if (single) {
      const float inv = lr[r] > 0.0f ? 1.0f / lr[r] : 0.0f;
#pragma unroll
      for (int i = 0; i < NT; ++i) vals[i] = lr[r] > 0.0f ? o[i][r] * inv : 0.0f;
      float* dst = a.out + ((int64_t)b * a.num_q_heads + hq) * D + d0;
#pragma unroll
      for (int i = 0; i < NT; i += 2) *reinterpret_cast<float2*>(dst + i) = make_float2(vals[i], vals[i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < NT; ++i) vals[i] = o[i][r];
      float* dst = a.ws_acc + (((int64_t)b * a.num_q_heads + hq) * a.n_split + split) * D + d0;
#pragma unroll
      for (int i = 0; i < NT; i += 2) *reinterpret_cast<float2*>(dst + i) = make_float2(vals[i], vals[i + 1]);
    }
  }
  if (!single && kg == 0 && head_on) {
    const int hq = qh_base + j;
    float* dst = a.ws_ml + (((int64_t)b * a.num_q_heads + hq) * a.n_split + split) * 2;
    *reinterpret_cast<float2*>(dst) = make_float2(m, l);
  }
}

// Combine the splits of each (sequence, q head): m* = max m_s,
// o = sum 2^(m_s - m*) acc_s / sum 2^(m_s - m*) l_s (log2 units).  Sequences with one
// split were finished by the split kernel; empty sequences get zeros.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.num_q_heads;
  const int lane = threadIdx.x;
  constexpr int PER = D / 64;
  float* dst = a.out + (int64_t)bh * D + lane * PER;
  const int L = min(a.seq_lens[b], a.max_blocks * a.pool.page_size);
  if (L <= 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) dst[i] = 0.0f;
    return;
  }
  const int hi = L - 1;
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int s0 = lo / a.split_keys, s1 = hi / a.split_keys;
  if (s0 == s1) return;
  const float* ml = a.ws_ml + (int64_t)bh * a.n_split * 2;
  const float* acc = a.ws_acc + (int64_t)bh * a.n_split * D + lane * PER;
  float mstar = -INFINITY;
  for (int s = s0; s <= s1; ++s) mstar = fmaxf(mstar, ml[2 * s]);
  if (mstar == -INFINITY) mstar = 0.0f;
  float o[PER] = {};
  float l = 0.0f;
  for (int s = s0; s <= s1; ++s) {
    const float w = fast_exp2(ml[2 * s] - mstar);
    l += w * ml[2 * s + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += w * acc[(int64_t)s * D + i];
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[i] = l > 0.0f ? o[i] * inv : 0.0f;
}

template <int KVT, int D>
hipError_t decode_dispatch_g(const DecodeArgs& a, hipStream_t s) {
  const int H = a.pool.num_kv_heads;
  const unsigned gy = (a.group == 8) ? H : (H + 1) / 2;
  const dim3 grid(a.n_split, gy, a.batch);
  switch (a.group) {
    case 8: hipLaunchKernelGGL((decode_split_kernel<KVT, D, 8>), grid, dim3(64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<KVT, D, 4>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<KVT, D, 2>), grid, dim3(64), 0, s, a); break;
    default: hipLaunchKernelGGL((decode_split_kernel<KVT, D, 1>), grid, dim3(64), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.batch * a.num_q_heads), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int KVT>
hipError_t decode_dispatch(const DecodeArgs& a, hipStream_t s) {
  if (a.pool.head_dim == 128) return decode_dispatch_g<KVT, 128>(a, s);
  return decode_dispatch_g<KVT, 64>(a, s);
}

}  // namespace

int decode_split_keys(int kv_dtype, int group, int page_size) {
  (void)group; (void)page_size;
  return kv_dtype == KV_FP8 ? 1024 : 512;
}

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  switch (kv_dtype) {
    case KV_F32: return decode_dispatch<KV_F32>(a, s);
    case KV_BF16: return decode_dispatch<KV_BF16>(a, s);
    default: return decode_dispatch<KV_FP8>(a, s);
  }
}

}  // namespace tl
