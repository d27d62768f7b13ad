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
#include <utility>

#include "tl_internal.h"

namespace tl {
namespace {

constexpr int TK = 32;  // keys per tile per slot

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <int KVT, int D>
struct Geo {
  using Tr = KvTraits<KVT>;
  static constexpr int X = Tr::X;
  static constexpr int NC = D / X;           // K chunks per key
  static constexpr int NT = D / 32;          // value MFMAs per key (d values per lane)
  static constexpr int VW = NT * Tr::BYTES;  // bytes of V per lane per key
  static constexpr int VWORDS = (VW + 3) / 4;
  static constexpr int NQ = D / 8;           // query registers per lane
};

template <int KVT, int D> struct KBuf { uint4 k[Geo<KVT, D>::NC]; v4f ks, vs; };
template <int KVT, int D> struct VBuf { uint32_t v[TK][Geo<KVT, D>::VWORDS]; };

// Page of a block, from the split's table entries held one per lane (lane i: block
// first_block + i).  Per-lane keys use ds_bpermute, wave-uniform keys v_readlane.
__device__ __forceinline__ int page_of_lane(int tab, int local) {
  return __builtin_amdgcn_ds_bpermute(local << 2, tab);
}
__device__ __forceinline__ int page_uniform(int tab, int local) { return __builtin_amdgcn_readlane(tab, local); }

#ifndef TL_DECODE_PREFETCH_BF16
#define TL_DECODE_PREFETCH_BF16 0
#endif
template <int KVT, int D> struct DecodePrefetch {
  static constexpr bool value = (KVT == KV_FP8) || (KVT == KV_BF16 && TL_DECODE_PREFETCH_BF16) || D == 64;
};

struct Split {
  int kvh, lo, hi, k_end, first_block, tab, lane;
};

// K chunks of this lane's key (kg*4 + j of the tile) and, for fp8, the K/V scales of
// keys kg*4 .. kg*4+3 (a group of 4 never straddles a page).
template <int KVT, int D>
__device__ __forceinline__ void load_k(KBuf<KVT, D>& t, const DecodeArgs& a, const Split& sp, int k0) {
  using GE = Geo<KVT, D>;
  const int S = a.pool.page_size, sh = a.pool.page_shift, H = a.pool.num_kv_heads;
  const int kg = (sp.lane >> 2) & 7, j = sp.lane & 3;
  const int key = clampi(k0 + kg * 4 + j, sp.lo, sp.hi);
  const int page = page_of_lane(sp.tab, clampi((key >> sh) - sp.first_block, 0, 63));
  const uint4* base = reinterpret_cast<const uint4*>(a.pool.k) + (((int64_t)page * H + sp.kvh) * GE::NC) * S +
                      (key & (S - 1));
#pragma unroll
  for (int c = 0; c < GE::NC; ++c) t.k[c] = base[(int64_t)c * S];
  if constexpr (KVT == KV_FP8) {
    const int g0 = clampi(k0 + kg * 4, sp.lo & ~3, sp.hi & ~3);
    const int pg = page_of_lane(sp.tab, clampi((g0 >> sh) - sp.first_block, 0, 63));
    const int64_t idx = ((int64_t)pg * H + sp.kvh) * S + (g0 & (S - 1));
    t.ks = *reinterpret_cast<const v4f*>(a.pool.k_scale + idx);
    t.vs = *reinterpret_cast<const v4f*>(a.pool.v_scale + idx);
  }
}

// V rows of the tile's 32 keys, NT values per lane per key.  Keys come in groups of 8
// that share a page (pages hold >= 8 keys), so each group needs one page lookup and
// its rows sit at fixed offsets.  A group wholly outside [lo, hi] reads some other
// rows of a valid page; those keys are never used.
template <int KVT, int D>
__device__ __forceinline__ void load_v(VBuf<KVT, D>& t, const DecodeArgs& a, const Split& sp, int k0) {
  using GE = Geo<KVT, D>;
  const int S = a.pool.page_size, sh = a.pool.page_shift, H = a.pool.num_kv_heads;
  const int d0 = (sp.lane & 31) * GE::NT;
#pragma unroll
  for (int g = 0; g < TK / 8; ++g) {
    const int kg0 = clampi(k0 + 8 * g, sp.lo & ~7, sp.hi & ~7);
    const int page = page_uniform(sp.tab, clampi((kg0 >> sh) - sp.first_block, 0, 63));
    const char* row = reinterpret_cast<const char*>(a.pool.v) +
                      ((((int64_t)page * H + sp.kvh) * S + (kg0 & (S - 1))) * D + d0) * GE::Tr::BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char* r = row + i * D * GE::Tr::BYTES;
      uint32_t* dst = t.v[8 * g + i];
      if constexpr (GE::VW == 16) {
        uint4 x = *reinterpret_cast<const uint4*>(r);
        dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
      } else if constexpr (GE::VW == 8) {
        uint2 x = *reinterpret_cast<const uint2*>(r);
        dst[0] = x.x; dst[1] = x.y;
      } else if constexpr (GE::VW == 4) {
        dst[0] = *reinterpret_cast<const uint32_t*>(r);
      } else {  // fp8 with D = 64: 2 bytes
        dst[0] = *reinterpret_cast<const uint16_t*>(r);
      }
    }
  }
}

// widen the NT value elements of key kk for this lane
template <int KVT, int D>
__device__ __forceinline__ void widen_v(const VBuf<KVT, D>& t, int kk, float* o) {
  using GE = Geo<KVT, D>;
  if constexpr (KVT == KV_F32) {
#pragma unroll
    for (int i = 0; i < GE::NT; ++i) o[i] = __uint_as_float(t.v[kk][i]);
  } else if constexpr (KVT == KV_BF16) {
#pragma unroll
    for (int i = 0; i < GE::NT / 2; ++i) { o[2 * i] = bf16_lo(t.v[kk][i]); o[2 * i + 1] = bf16_hi(t.v[kk][i]); }
  } else {
    if constexpr (GE::NT == 4) {
      fp8x4_to_f32(t.v[kk][0], o);
    } else {
      typedef float v2f __attribute__((ext_vector_type(2)));
      v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)t.v[kk][0], false);
      o[0] = lo[0]; o[1] = lo[1];
    }
  }
}

// values: O[i] += P(key KG*4 + r) * V(key, d(lane, i)), P broadcast from block KG of the slot
template <int KVT, int D, int KG, bool GUARD>
__device__ __forceinline__ void pv_group(const VBuf<KVT, D>& t, const float* pv, v4f* o, int kk_lo, int kk_hi) {
  using GE = Geo<KVT, D>;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kk = KG * 4 + r;
    if (GUARD && (kk < kk_lo || kk > kk_hi)) continue;  // wave-uniform
    float vv[GE::NT];
    widen_v<KVT, D>(t, kk, vv);
#pragma unroll
    for (int i = 0; i < GE::NT; ++i) o[i] = __builtin_amdgcn_mfma_f32_4x4x1f32(pv[r], vv[i], o[i], 3, KG, 0);
  }
}

template <int KVT, int D, bool GUARD>
__device__ __forceinline__ void pv_tile(const VBuf<KVT, D>& t, const float* pv, v4f* o, int kk_lo, int kk_hi) {
  pv_group<KVT, D, 0, GUARD>(t, pv, o, kk_lo, kk_hi);
  pv_group<KVT, D, 1, GUARD>(t, pv, o, kk_lo, kk_hi);
  pv_group<KVT, D, 2, GUARD>(t, pv, o, kk_lo, kk_hi);
  pv_group<KVT, D, 3, GUARD>(t, pv, o, kk_lo, kk_hi);
  pv_group<KVT, D, 4, GUARD>(t, pv, o, kk_lo, kk_hi);
  pv_group<KVT, D, 5, GUARD>(t, pv, o, kk_lo, kk_hi);
  pv_group<KVT, D, 6, GUARD>(t, pv, o, kk_lo, kk_hi);
  pv_group<KVT, D, 7, GUARD>(t, pv, o, kk_lo, kk_hi);
}

// scores: S[head i][key] = sum_d Q[i][d] K[key][d].  A = Q broadcast from block d%8
// (register d/8 of that block holds d), B = this lane's K value.  Result: lane
// (kg, j) register i = S[head i][key kg*4 + j]; two chains over d.  The d loop is
// unrolled through parameter packs because CBSZ/ABID must be constants.
template <int KVT, int D, int C, int... Es>
__device__ __forceinline__ void qk_chunk(const uint4& raw, const float* q, v4f& s0, v4f& s1,
                                         std::integer_sequence<int, Es...>) {
  constexpr int X = Geo<KVT, D>::X;
  float kv[X];
  widen_chunk<KVT>(raw, kv);
  ((Es % 2 == 0
        ? (void)(s0 = __builtin_amdgcn_mfma_f32_4x4x1f32(q[(C * X + Es) >> 3], kv[Es], s0, 3, (C * X + Es) & 7, 0))
        : (void)(s1 = __builtin_amdgcn_mfma_f32_4x4x1f32(q[(C * X + Es) >> 3], kv[Es], s1, 3, (C * X + Es) & 7, 0))),
   ...);
}

template <int KVT, int D, int... Cs>
__device__ __forceinline__ v4f qk_all(const KBuf<KVT, D>& kb, const float* q, std::integer_sequence<int, Cs...>) {
  v4f s0 = v4f{0, 0, 0, 0}, s1 = v4f{0, 0, 0, 0};
  (qk_chunk<KVT, D, Cs>(kb.k[Cs], q, s0, s1, std::make_integer_sequence<int, Geo<KVT, D>::X>{}), ...);
  return s0 + s1;
}

template <int KVT, int D>
__device__ __forceinline__ v4f qk_tile(const KBuf<KVT, D>& kb, const float* q) {
  return qk_all<KVT, D>(kb, q, std::make_integer_sequence<int, Geo<KVT, D>::NC>{});
}

// 4x4 transpose inside each quad of lanes: register r of lane j <- register j of lane r
__device__ __forceinline__ v4f quad_transpose(v4f x, int j) {
  const bool odd = j & 1, hi = j & 2;
  auto swap1 = [](float v) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)); };
  auto swap2 = [](float v) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)); };
  const float a = swap1(x[1]), b = swap1(x[0]), c = swap1(x[3]), d = swap1(x[2]);
  v4f z;
  z[0] = odd ? a : x[0];
  z[1] = odd ? x[1] : b;
  z[2] = odd ? c : x[2];
  z[3] = odd ? x[3] : d;
  const float e = swap2(z[2]), f = swap2(z[0]), g = swap2(z[3]), h = swap2(z[1]);
  v4f y;
  y[0] = hi ? e : z[0];
  y[2] = hi ? z[2] : f;
  y[1] = hi ? g : z[1];
  y[3] = hi ? z[3] : h;
  return y;
}
// One tile: issue this tile's V rows and the next tile's K chunks, then scores on the
// current K, online softmax, and values.
template <int KVT, int D, bool PF>
__device__ __forceinline__ void decode_tile(const DecodeArgs& a, const Split& sp, KBuf<KVT, D>& kc,
                                            KBuf<KVT, D>& kn, VBuf<KVT, D>& vt, int k0, const float* q, v4f* o,
                                            float& m, float& l) {
  using GE = Geo<KVT, D>;
  const int kg = (sp.lane >> 2) & 7, j = sp.lane & 3;
  if constexpr (!PF) load_k<KVT, D>(kc, a, sp, k0);
  load_v<KVT, D>(vt, a, sp, k0);
  if constexpr (PF) {
    if (k0 + TK <= sp.k_end) load_k<KVT, D>(kn, a, sp, k0 + TK);
  }

  // ---- scores, then lane (kg, j) register r = S[head j][key kg*4 + r]
  v4f sc = quad_transpose(qk_tile<KVT, D>(kc, q), j);

  // ---- mask, online softmax (per head = per lane j within the slot)
  float s[4], tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = k0 + kg * 4 + r;
    const bool valid = key >= sp.lo && key <= sp.k_end;
    float x = sc[r];
    if constexpr (KVT == KV_FP8) x *= kc.ks[r];
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
    if constexpr (KVT == KV_FP8) pv[r] = (s[r] == -INFINITY) ? 0.0f : p[r] * kc.vs[r];
    else pv[r] = p[r];
  }
  // rescale the value accumulators: register r of a quad holds head r of the slot
  const float a0 = quad_bcast<0>(alpha), a1 = quad_bcast<1>(alpha);
  const float a2 = quad_bcast<2>(alpha), a3 = quad_bcast<3>(alpha);
#pragma unroll
  for (int i = 0; i < GE::NT; ++i) { o[i][0] *= a0; o[i][1] *= a1; o[i][2] *= a2; o[i][3] *= a3; }

  // ---- values; keys outside [lo, k_end] are skipped (their V rows are not theirs)
  const int kk_lo = max(sp.lo - k0, 0), kk_hi = min(sp.k_end - k0, TK - 1);
  if (kk_lo == 0 && kk_hi == TK - 1) pv_tile<KVT, D, false>(vt, pv, o, 0, TK - 1);
  else pv_tile<KVT, D, true>(vt, pv, o, kk_lo, kk_hi);
}

template <int KVT, int D, int G>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using GE = Geo<KVT, D>;
  constexpr int NT = GE::NT, NQ = GE::NQ;
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

  Split sp;
  sp.kvh = kvh; sp.lo = lo; sp.hi = hi; sp.k_end = k_end; sp.lane = lane;
  // the split's block-table entries, one per lane (a split spans at most 64 pages)
  sp.first_block = k_begin >> a.pool.page_shift;
  {
    const int last_block = k_end >> a.pool.page_shift;
    const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
    sp.tab = clampi(table[min(sp.first_block + lane, last_block)], 0, a.pool.num_pages - 1);
  }

  // queries: register t of lane (slot, kg, j) holds Q[head j][d = 8t + kg] * scale * log2(e)
  float q[NQ];
  {
    const float* qp = a.q + ((int64_t)b * a.num_q_heads + qh_base + j) * D + kg;
#pragma unroll
    for (int t = 0; t < NQ; ++t) q[t] = head_on ? qp[8 * t] * a.qscale : 0.0f;
  }

  v4f o[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) o[i] = v4f{0, 0, 0, 0};
  float m = -INFINITY, l = 0.0f;

  // K of the next tile is prefetched into a second buffer where registers allow it
  // (fp8); otherwise each tile loads its own K and relies on more waves per SIMD.
  constexpr bool PF = DecodePrefetch<KVT, D>::value;
  KBuf<KVT, D> kA, kB;
  VBuf<KVT, D> vt;
  if constexpr (PF) load_k<KVT, D>(kA, a, sp, k_begin);
  for (int k0 = k_begin;;) {
    decode_tile<KVT, D, PF>(a, sp, kA, kB, vt, k0, q, o, m, l);
    k0 += TK;
    if (k0 > k_end) break;
    decode_tile<KVT, D, PF>(a, sp, kB, kA, vt, k0, q, o, m, l);
    k0 += TK;
    if (k0 > k_end) break;
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
  (void)group;
  const int want = kv_dtype == KV_FP8 ? 1024 : 512;
  return want < 64 * page_size ? want : 64 * page_size;  // a split spans at most 64 pages
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
