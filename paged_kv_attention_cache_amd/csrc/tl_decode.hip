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
#include <mutex>
#include <type_traits>
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

// How far ahead a wave loads: 0 = each tile loads its own K and V; 1 = the next
// tile's K is loaded with this tile's V; 2 = the next tile's K and V are loaded while
// this tile computes.  Chosen by what fits in the register budget (1-byte tiles are
// small; bf16 and f32 tiles at D = 128 rely on more waves per SIMD instead).  For
// int8 at D = 128, measured on the c2 layer: 0 193 us, 1 145 us, 2 168 us (spills).
template <int KVT, int D, int G> struct DecodePrefetch {
  static constexpr int value = (KVT == KV_INT8 && D == 128) ? 1
                             : (kv_fp8(KVT) && D == 128 && G == 8) ? 1 : (D == 64 ? 1 : 0);
};

// tab: the split's table entry first_block + lane; tab2 (int8 tile, whose splits span
// up to 128 pages): entry first_block + 64 + lane
struct Split {
  int kvh, lo, hi, k_end, first_block, tab, tab2, lane;
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
  for (int c = 0; c < GE::NC; ++c) t.k[c] = stream_load(base + (int64_t)c * S);
  if constexpr (kv_scaled(KVT)) {
    const int g0 = clampi(k0 + kg * 4, sp.lo & ~3, sp.hi & ~3);
    const int pg = page_of_lane(sp.tab, clampi((g0 >> sh) - sp.first_block, 0, 63));
    const int64_t idx = ((int64_t)pg * H + sp.kvh) * S + (g0 & (S - 1));
    t.ks = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.pool.k_scale + idx));
    t.vs = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.pool.v_scale + idx));
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
        const uint4 x = stream_load(reinterpret_cast<const uint4*>(r));
        dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
      } else if constexpr (GE::VW == 8) {
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        const u2 x = __builtin_nontemporal_load(reinterpret_cast<const u2*>(r));
        dst[0] = x[0]; dst[1] = x[1];
      } else if constexpr (GE::VW == 4) {
        dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(r));
      } else {  // fp8 with D = 64: 2 bytes
        dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(r));
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
  } else if constexpr (KVT == KV_INT8) {
#pragma unroll
    for (int i = 0; i < GE::NT; ++i) o[i] = (float)(int8_t)(t.v[kk][0] >> (8 * i));
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
struct NoHook { __device__ __forceinline__ void operator()() const {} };

template <int KVT, int D, int PF, typename Hook = NoHook>
__device__ __forceinline__ void decode_tile(const DecodeArgs& a, const Split& sp, KBuf<KVT, D>& kc,
                                            KBuf<KVT, D>& kn, VBuf<KVT, D>& vt, VBuf<KVT, D>& vn, int k0,
                                            int k_next, const float* q, v4f* o, float& m, float& l,
                                            Hook hook = Hook()) {
  using GE = Geo<KVT, D>;
  const int kg = (sp.lane >> 2) & 7, j = sp.lane & 3;
  if constexpr (PF == 0) {
    load_k<KVT, D>(kc, a, sp, k0);
    load_v<KVT, D>(vt, a, sp, k0);
  } else if constexpr (PF == 1) {
    load_v<KVT, D>(vt, a, sp, k0);
    if (k_next <= sp.k_end) load_k<KVT, D>(kn, a, sp, k_next);
  } else {
    if (k_next <= sp.k_end) {
      load_k<KVT, D>(kn, a, sp, k_next);
      load_v<KVT, D>(vn, a, sp, k_next);
    }
  }
  hook();  // loads for later work, issued behind this tile's own

  // ---- scores, then lane (kg, j) register r = S[head j][key kg*4 + r]
  v4f sc = quad_transpose(qk_tile<KVT, D>(kc, q), j);

  // ---- mask, online softmax (per head = per lane j within the slot)
  float s[4], tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = k0 + kg * 4 + r;
    const bool valid = key >= sp.lo && key <= sp.k_end;
    float x = sc[r];
    if constexpr (kv_scaled(KVT)) x *= kc.ks[r];
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
    if constexpr (kv_scaled(KVT)) pv[r] = (s[r] == -INFINITY) ? 0.0f : p[r] * kc.vs[r];
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


// ------------------------------------------------ fp8, D = 128, G = 8: exact bf16 split
// For the fp8 pool with 8 query heads per KV head, both dots run on
// v_mfma_f32_16x16x32_bf16 without changing the arithmetic: every fp8 K and V value
// is exactly a bf16, and each f32 operand on the other side (the scaled query, the
// scaled probability) is split exactly into three bf16 terms, hi + mid + lo (each the
// truncation of what remains, 8 significant bits at a time).  The products of bf16
// terms are exact in f32 and the matrix core sums them in f32, so a dot is still f32
// operands, f32 products and f32 sums, only summed in a different order.
//
// Per wave and 32-key tile of one KV head (lane l, c = l % 16, g = l / 16):
//   scores  S^T[key, col] = sum_d K[key, d] Q3[col, d]: two 16-key halves x two
//           column tiles (columns: hi and mid of heads 0-7, then lo of heads 0-7 and
//           8 zero columns) x four 32-wide d steps = 16 MFMAs.  In step s the MFMA
//           index k = 8g + e stands for d = 32g + 8s + e, so a lane's K bytes for
//           the four steps are its key's two contiguous 16-byte chunks 2g, 2g+1.
//           Lane l then holds, for head c (c < 8), keys 16*h + 4g + r of the tile
//           (h = half, r = 0..3).
//   values  O3[row, d] += sum_key P3[row, key] V[key, d]: rows are hi and mid of
//           heads 0-7 (tile 0) and lo (tile 1); d = 8c + n for d tile n = 0..7; the
//           key order of the sum is that of the score lanes (key 16*(e/4) + 4g + e%4
//           for k = 8g + e), so P stays in the lane that computed it: 16 MFMAs.
// Per lane per tile: 4 K loads of 16 bytes, 8 V loads of 8 bytes and 4 scale loads;
// no value is loaded twice.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct XBuf {
  u32x4 k[2][2];  // [half][chunk]: 16 fp8 of key 16*half + c at d 32g + 16j .. +15
  u32x2 v[8];     // [e]: 8 fp8 of key 16*(e/4) + 4g + e%4 at d 8c .. 8c+7
  v4f ks[2], vs[2];  // [half]: scales of keys 16*half + 4g .. +3
};

__device__ __forceinline__ uint32_t bf16_pair_of(float a, float b) {
  // a, b are exact bf16 values (low 16 bits zero): pack them as (a, b)
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ __forceinline__ float trunc_bf16(float x) { return __uint_as_float(__float_as_uint(x) & 0xFFFF0000u); }
// x = hi + mid + lo exactly, each a bf16 value
__device__ __forceinline__ void split3(float x, float& hi, float& mid, float& lo) {
  hi = trunc_bf16(x);
  const float r1 = x - hi;
  mid = trunc_bf16(r1);
  lo = trunc_bf16(r1 - mid);
}
// lane i of each 16-lane row receives lane i ^ 8 (DPP row rotate by 8)
__device__ __forceinline__ uint32_t ror8(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false); }
__device__ __forceinline__ float ror8f(float v) { return __uint_as_float(ror8(__float_as_uint(v))); }

// two fp8 codes (bytes 2W, 2W+1 of x) -> packed bf16 pair, exact
template <bool W>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, W);
  return __builtin_bit_cast(uint32_t, r);
}

// Parts of a tile's operands, loaded separately so each can be refilled for the next
// tile as soon as this tile has consumed it.
struct XHalf { int64_t ph; int hk0; };
__device__ __forceinline__ XHalf xhalf(const DecodeArgs& a, const Split& sp, int k0, int h) {
  // a 16-key half never straddles a page (pages hold >= 16 keys here)
  XHalf r;
  r.hk0 = clampi(k0 + 16 * h, sp.lo & ~15, sp.hi & ~15);
  const int page = page_uniform(sp.tab, clampi((r.hk0 >> a.pool.page_shift) - sp.first_block, 0, 63));
  r.ph = (int64_t)page * a.pool.num_kv_heads + sp.kvh;
  return r;
}
__device__ __forceinline__ void xload_k(XBuf& t, const DecodeArgs& a, const Split& sp, int k0) {
  constexpr int NC = 128 / 16;
  const int S = a.pool.page_size, c = sp.lane & 15, g = sp.lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const XHalf x = xhalf(a, sp, k0, h);
    // key clamped into [lo, hi]; chunks 2g and 2g + 1 (d 32g .. 32g + 31)
    const int key = clampi(x.hk0 + c, sp.lo, sp.hi);
    const uint4* kb = reinterpret_cast<const uint4*>(a.pool.k) + (x.ph * NC + 2 * g) * S + (key & (S - 1));
#pragma unroll
    for (int j = 0; j < 2; ++j) t.k[h][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)j * S));
  }
}
__device__ __forceinline__ void xload_scales(XBuf& t, const DecodeArgs& a, const Split& sp, int k0, bool kside) {
  const int S = a.pool.page_size, g = sp.lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const XHalf x = xhalf(a, sp, k0, h);
    const int g0 = clampi(x.hk0 + 4 * g, sp.lo & ~3, sp.hi & ~3);
    const int64_t si = x.ph * S + (g0 & (S - 1));
    if (kside) t.ks[h] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.pool.k_scale + si));
    else t.vs[h] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.pool.v_scale + si));
  }
}
__device__ __forceinline__ void xload_v(XBuf& t, const DecodeArgs& a, const Split& sp, int k0) {
  constexpr int D = 128;
  const int S = a.pool.page_size, c = sp.lane & 15, g = sp.lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const XHalf x = xhalf(a, sp, k0, h);
    // rows of keys hk0 + 4g + r, clamped into [lo, hi]; bytes 8c .. 8c+7
    const int rlo = sp.lo - x.hk0, rhi = sp.hi - x.hk0;
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(a.pool.v) + (x.ph * S + (x.hk0 & (S - 1))) * D + 8 * c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = min(max(4 * g + r, rlo), rhi);
      t.v[4 * h + r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vb + (int64_t)row * D));
    }
  }
}
template <bool SC>
__device__ __forceinline__ void xload(XBuf& t, const DecodeArgs& a, const Split& sp, int k0) {
  xload_k(t, a, sp, k0);
  if constexpr (SC) {
    xload_scales(t, a, sp, k0, true);
    xload_scales(t, a, sp, k0, false);
  }
  xload_v(t, a, sp, k0);
}

// One 32-key tile on the operands in t; each part of t is reloaded with the next
// tile's as soon as it has been used.  qs: this wave's Q3 operands in LDS
// ([col tile][d step][lane]); o: [row tile][d tile].  The running max m only moves
// when a tile's max exceeds it by more than 8 (log2 units, a factor 2^8), so the
// accumulators are rarely rescaled; probabilities then stay below 2^8.
template <bool SC, typename Hook = NoHook>
__device__ __forceinline__ void xtile(const DecodeArgs& a, const Split& sp, XBuf& t, int k0, int k_next,
                                      const bf16x8* qs, v4f (&o)[2][8], float& m, float& l, Hook hook = Hook()) {
  const int c = sp.lane & 15, g = sp.lane >> 4;
  const bool more = k_next <= sp.k_end;
  // ---- scores
  v4f sc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v4f t0 = v4f{0, 0, 0, 0}, t1 = v4f{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t d0 = t.k[h][st >> 1][2 * (st & 1)], d1 = t.k[h][st >> 1][2 * (st & 1) + 1];
      uint32_t w[4];
      w[0] = fp8x2_to_bf16x2<false>(d0);
      w[1] = fp8x2_to_bf16x2<true>(d0);
      w[2] = fp8x2_to_bf16x2<false>(d1);
      w[3] = fp8x2_to_bf16x2<true>(d1);
      const bf16x8 ka = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qs[(0 * 4 + st) * 64 + sp.lane], t0, 0, 0, 0);
      t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qs[(1 * 4 + st) * 64 + sp.lane], t1, 0, 0, 0);
    }
    // head c: hi (column c) + mid (column c + 8) + lo (column c of tile 1)
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[h][r] = (t0[r] + ror8f(t0[r])) + t1[r];
  }
  if (more) xload_k(t, a, sp, k_next);
  // ---- mask, online softmax for head c over the wave's 32 keys
  float s8[8], tmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int h = e >> 2, r = e & 3;
    const int key = k0 + 16 * h + 4 * g + r;
    const bool valid = key >= sp.lo && key <= sp.k_end;
    s8[e] = valid ? (SC ? sc[h][r] * t.ks[h][r] : sc[h][r]) : -INFINITY;
    tmax = fmaxf(tmax, s8[e]);
  }
  if (SC && more) xload_scales(t, a, sp, k_next, true);
  tmax = wave_xor_max(tmax, 16);
  tmax = wave_xor_max(tmax, 32);
  // lazy max: keep m unless this tile exceeds it by more than 8 (or m is unset)
  const float m_new = (m == -INFINITY || tmax > m + 8.0f) ? tmax : m;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = (m == -INFINITY) ? 1.0f : fast_exp2(m - m_use);  // o and l are 0 while m is unset
  float psum = 0.0f;
  float ph[8], pm[8], pl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = fast_exp2(s8[e] - m_use);
    psum += p;
    const float pv = (s8[e] == -INFINITY) ? 0.0f : (SC ? p * t.vs[e >> 2][e & 3] : p);
    split3(pv, ph[e], pm[e], pl[e]);
  }
  if (SC && more) xload_scales(t, a, sp, k_next, false);
  l = l * alpha + psum;
  m = m_new;
  // ---- A operands of the value product: rows hi / mid (tile 0) and lo (tile 1)
  uint32_t a0[4], a1[4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const uint32_t hi2 = bf16_pair_of(ph[2 * qd], ph[2 * qd + 1]);
    const uint32_t mid2 = ror8(bf16_pair_of(pm[2 * qd], pm[2 * qd + 1]));
    const uint32_t lo2 = bf16_pair_of(pl[2 * qd], pl[2 * qd + 1]);
    a0[qd] = c < 8 ? hi2 : mid2;
    a1[qd] = c < 8 ? lo2 : 0u;
  }
  const bf16x8 pa0 = __builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a0[2], a0[3]});
  const bf16x8 pa1 = __builtin_bit_cast(bf16x8, u32x4{a1[0], a1[1], a1[2], a1[3]});
  // ---- rescale: accumulator row 4g + r belongs to head 4(g % 2) + r
  if (__any(c < 8 && alpha != 1.0f)) {
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * (g & 1) + r, 64);
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) { o[0][n][r] *= ar[r]; o[1][n][r] *= ar[r]; }
  }
  // ---- values: B operand of d tile n = V[key(8g + e)][8c + n] for e = 0..7
#pragma unroll
  for (int np = 0; np < 4; ++np) {  // d tiles 2np, 2np + 1 share one byte gather
    const int word = np >> 1, b0 = (np & 1) * 2;
    const uint32_t sel = (uint32_t)b0 | ((uint32_t)(b0 + 4) << 8) | ((uint32_t)(b0 + 1) << 16) | ((uint32_t)(b0 + 5) << 24);
    uint32_t lo4[4], hi4[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const uint32_t x = __builtin_amdgcn_perm(t.v[2 * qd + 1][word], t.v[2 * qd][word], sel);
      lo4[qd] = fp8x2_to_bf16x2<false>(x);  // keys 2qd, 2qd+1 at d 8c + 2np
      hi4[qd] = fp8x2_to_bf16x2<true>(x);   // same keys at d 8c + 2np + 1
    }
    const bf16x8 vb0 = __builtin_bit_cast(bf16x8, u32x4{lo4[0], lo4[1], lo4[2], lo4[3]});
    const bf16x8 vb1 = __builtin_bit_cast(bf16x8, u32x4{hi4[0], hi4[1], hi4[2], hi4[3]});
    o[0][2 * np] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa0, vb0, o[0][2 * np], 0, 0, 0);
    o[1][2 * np] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa1, vb0, o[1][2 * np], 0, 0, 0);
    o[0][2 * np + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa0, vb1, o[0][2 * np + 1], 0, 0, 0);
    o[1][2 * np + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa1, vb1, o[1][2 * np + 1], 0, 0, 0);
  }
  if (more) xload_v(t, a, sp, k_next);
  hook();
}

// Q of an item as the B operands of the score product: for column tile t and d step
// s, lane l holds column c = l % 16 at d = 32g + 8s + e: tile 0 column c < 8 = hi of
// head c, c >= 8 = mid of head c - 8; tile 1 column c < 8 = lo of head c, else 0.
// The operands are shared by the workgroup's waves; each builds one step st from the
// 8 raw values qraw = Q[head c % 8][32g + 8st .. +7].
__device__ __forceinline__ void xqueries(const float (&qraw)[8], float qscale, int lane, int st, bf16x8* qs) {
  const int c = lane & 15;
  uint32_t w0[4], w1[4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    float h0, m0, l0, h1, m1, l1;
    split3(qraw[2 * qd] * qscale, h0, m0, l0);
    split3(qraw[2 * qd + 1] * qscale, h1, m1, l1);
    w0[qd] = c < 8 ? bf16_pair_of(h0, h1) : bf16_pair_of(m0, m1);
    w1[qd] = c < 8 ? bf16_pair_of(l0, l1) : 0u;
  }
  qs[(0 * 4 + st) * 64 + lane] = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w0[2], w0[3]});
  qs[(1 * 4 + st) * 64 + lane] = __builtin_bit_cast(bf16x8, u32x4{w1[0], w1[1], w1[2], w1[3]});
}

// ---------------------------------------------- bf16 KV, D = 128, G = 4: exact bf16 split
// The same arithmetic for a KV head with 4 query heads, one KV head per wave.  Every
// stored K and V value is a bf16, and the f32 operand on the other side is split
// exactly into hi + mid + lo bf16 terms.  The 4 heads' 3 terms fill 12 of a tile's 16 columns, so one column tile
// holds them all.  Per 32-key tile (lane l, c = l % 16, g = l / 16):
//   scores  S^T[key, col] = sum_d K[key, d] Q3[col, d] for each 16-key half over four
//           32-wide d steps: 8 MFMAs.  Column c is term c / 4 (hi, mid, lo; 3 = zero) of
//           head c % 4; lane (c, g) gets keys 16h + 4g + r of column c.  A butterfly
//           over lanes c ^ 4 and c ^ 8 adds the columns c % 4 + 4t, leaving in every
//           lane head c % 4's whole score for its 8 keys.
//   values  O3[row, d] += sum_key P3[row, key] V[key, d], d = 8c + n in d tile n: 8
//           MFMAs.  Row c is term c / 4 of head c % 4's probability, which lane (c, g)
//           computed itself for exactly the keys its operand needs (k = 8g + e stands for
//           key 16(e / 4) + 4g + e % 4, as in the score lanes).  Accumulator row 4g + r is
//           term g of head r.
// In score step s, k = 8g + e stands for d = 32g + 8s + e (as for G = 8): a lane's K
// bytes are its key's d 32g .. 32g + 31, the bf16 chunks 4g .. 4g + 3, each of which is
// the A operand of one step as loaded.
struct X4Buf {
  u32x4 k[2][4];      // [half][step]: key 16 * half + c, chunk 4g + step
  uint32_t v[8][4];   // [e]: key 16(e/4) + 4g + e%4 at d 8c .. 8c + 7
};

__device__ __forceinline__ void x4load_k(X4Buf& t, const DecodeArgs& a, const Split& sp, int k0) {
  constexpr int NC = 128 / 8;
  const int S = a.pool.page_size, c = sp.lane & 15, g = sp.lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const XHalf x = xhalf(a, sp, k0, h);
    const int key = clampi(x.hk0 + c, sp.lo, sp.hi);
    const uint4* kb = reinterpret_cast<const uint4*>(a.pool.k) + (x.ph * NC + 4 * g) * S + (key & (S - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.k[h][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)j * S));
  }
}

__device__ __forceinline__ void x4load_v(X4Buf& t, const DecodeArgs& a, const Split& sp, int k0) {
  constexpr int D = 128;
  const int S = a.pool.page_size, c = sp.lane & 15, g = sp.lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const XHalf x = xhalf(a, sp, k0, h);
    // rows of keys hk0 + 4g + r, clamped into [lo, hi]; d 8c .. 8c + 7
    const int rlo = sp.lo - x.hk0, rhi = sp.hi - x.hk0;
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.pool.v) + (x.ph * S + (x.hk0 & (S - 1))) * D + 8 * c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = min(max(4 * g + r, rlo), rhi);
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (int64_t)row * D));
      t.v[4 * h + r][0] = w[0]; t.v[4 * h + r][1] = w[1]; t.v[4 * h + r][2] = w[2]; t.v[4 * h + r][3] = w[3];
    }
  }
}

// One 32-key tile on the operands in t (each part reloaded with the next tile's once
// used); qs: this item's Q3 operands in LDS ([d step][lane]); o: [d tile].  Lazy
// running max as in xtile.
template <typename Hook = NoHook>
__device__ __forceinline__ void xtile4(const DecodeArgs& a, const Split& sp, X4Buf& t, int k0, int k_next,
                                       const bf16x8* qs, v4f (&o)[8], float& m, float& l, Hook hook = Hook()) {
  const int c = sp.lane & 15, g = sp.lane >> 4, term = c >> 2;
  const bool more = k_next <= sp.k_end;
  // work for later (the next item's claim) goes out first, so its round trip overlaps
  // this tile's arithmetic (measured: c2 -1%; at the end of the G = 8 tile instead,
  // where the start cost c5 5%)
  hook();
  // ---- scores; then every lane holds head c % 4's score of keys 16h + 4g + r
  v4f sc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v4f acc = v4f{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[h][st]), qs[st * 64 + sp.lane],
                                                    acc, 0, 0, 0);
    // The four columns of a head are added as a butterfly over lanes c ^ 4, then c ^ 8
    // (within a 16-lane row the rotation by 8 is the xor): every lane of the head adds
    // the same two numbers at each level, so all four hold bit-identical scores.  They
    // then agree on the max, the probabilities and their hi / mid / lo split, so the
    // three terms of one probability, taken from different lanes, add up to it exactly.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = acc[r] + __shfl_xor(acc[r], 4, 64);
      sc[h][r] = x + ror8f(x);
    }
  }
  if (more) x4load_k(t, a, sp, k_next);
  // ---- mask, online softmax for head c % 4 over the wave's 32 keys
  float s8[8], tmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int h = e >> 2, r = e & 3;
    const int key = k0 + 16 * h + 4 * g + r;
    const bool valid = key >= sp.lo && key <= sp.k_end;
    s8[e] = valid ? sc[h][r] : -INFINITY;
    tmax = fmaxf(tmax, s8[e]);
  }
  tmax = wave_xor_max(tmax, 16);
  tmax = wave_xor_max(tmax, 32);
  const float m_new = (m == -INFINITY || tmax > m + 8.0f) ? tmax : m;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = (m == -INFINITY) ? 1.0f : fast_exp2(m - m_use);
  float psum = 0.0f, pt[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = fast_exp2(s8[e] - m_use);
    psum += p;
    float hi, mid, lo;
    split3(p, hi, mid, lo);
    pt[e] = term == 0 ? hi : (term == 1 ? mid : (term == 2 ? lo : 0.0f));
  }
  l = l * alpha + psum;
  m = m_new;
  const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{bf16_pair_of(pt[0], pt[1]), bf16_pair_of(pt[2], pt[3]),
                                                     bf16_pair_of(pt[4], pt[5]), bf16_pair_of(pt[6], pt[7])});
  // ---- rescale: accumulator row 4g + r belongs to head r
  if (__any(alpha != 1.0f)) {
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, r, 64);
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[n][r] *= ar[r];
  }
  // ---- values: B operand of d tile n = V[key(8g + e)][8c + n] for e = 0..7, the n-th
  // bf16 of each key's 8 (high or low half of word n / 2)
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) w[qd] = __builtin_amdgcn_perm(t.v[2 * qd + 1][n >> 1], t.v[2 * qd][n >> 1], sel);
    o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]}), o[n],
                                                   0, 0, 0);
  }
  if (more) x4load_v(t, a, sp, k_next);
}

// Q of an item as the B operand of the G = 4 score product: for d step st, lane l
// holds column c = l % 16 at d = 32g + 8st + e: term c / 4 (hi, mid, lo, then zero) of
// head c % 4.  Each wave builds one step st from qraw = Q[head c % 4][32g + 8st .. +7].
__device__ __forceinline__ void xqueries4(const float (&qraw)[8], float qscale, int lane, int st, bf16x8* qs) {
  const int term = (lane & 15) >> 2;
  uint32_t w[4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    float h0, m0, l0, h1, m1, l1;
    split3(qraw[2 * qd] * qscale, h0, m0, l0);
    split3(qraw[2 * qd + 1] * qscale, h1, m1, l1);
    w[qd] = term == 0 ? bf16_pair_of(h0, h1) : (term == 1 ? bf16_pair_of(m0, m1) : (term == 2 ? bf16_pair_of(l0, l1) : 0u));
  }
  qs[st * 64 + lane] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// ------------------------------------- int8 KV, D = 128, G = 4: integer matrix cores
// The stored int8 codes are the operands of v_mfma_i32_16x16x64_i8 as loaded.  The f32
// operand on the other side (the scaled queries; a head's probabilities times the V
// scales) is written as a power of two and four 7-bit integer limbs:
//   y = sign * 2^(E - 6) * (c0 + c1 2^-7 + c2 2^-14 + c3 2^-21),  c0 < 64, c1..c3 < 128,
// where 2^E bounds |y| over a row (a query head over d; a head's tile of probabilities)
// and c0..c3 are the bits of the integer truncation of |y| 2^(27 - E), which drops less
// than 2^(E - 27) per value.  Both products are then exact integer sums: at most
// 128 * 127 * 127 (scores) or 64 * 127 * 127 (values), below 2^24, so they convert to
// f32 exactly, and each limb's sum is scaled by its power of two.  One 64-key tile per
// wave (lane l, c = l % 16, g = l / 16, t = c / 4, head h = c % 4):
//   scores  for each 16-key quarter qr: S[key, col] = sum_d K[key, d] Ql[col, d] over two
//           64-wide d steps (8 MFMAs per tile).  Column c is limb t of head h; lane (c, g)
//           gets keys 16qr + 4g + r and weights its sums by 2^(e_h - 6 - 7t).  A
//           reduce-scatter over the head's four limb lanes (c ^ 4, then c ^ 8) leaves in
//           lane (c, g) the whole score of the keys of quarter t, 16t + 4g + r: each lane
//           runs the softmax on its own 4 keys, and each key's score is summed in one lane.
//   values  Ol[row, d] = sum_key Pl[row, key] V[key, d], d = 8c + n for d tile n (8
//           MFMAs).  Row c is limb t of head h's p * v_scale over the lane group's 16 keys
//           (k = 16g + 4qr + r stands for key 16qr + 4g + r): the lane owning quarter qr
//           cuts its 4 keys into 4 limbs, and a transpose over the four limb lanes hands
//           limb t of every quarter to lane t.  Result row 4g + r (limb g of head r) is
//           weighted by 2^(E_r - 6 - 7g) and added to the f32 accumulator, so the sum
//           over lane groups at the end adds the limbs.
// In score step s, k = 16g + j stands for d = 16(4s + g) + j: a lane's K chunk 4s + g is
// its A operand as loaded.  V rows are loaded 8 bytes (d 8c .. 8c + 7) per key; the B
// operand of d tile n takes byte n of each of the lane's 16 keys, a 4 x 4 byte transpose
// per quarter and half row.  Codes of keys outside [lo, hi] are read from the same
// page (an int8 code is never NaN) and meet zero limbs or a masked score.  Scales are
// read in 4-key groups clamped into [lo, hi] rounded out to 4; a group's keys outside
// [lo, hi] may hold scales never written, so a masked key's K scale never reaches a
// used score and its probability stays exactly 0, not 0 times its V scale.
struct IBuf {
  u32x4 k[4][2];  // [quarter][step]: key 16 * quarter + c, chunk 4 * step + g
  uint32_t v[4][4][2];  // [quarter][r]: key 16 * quarter + 4g + r at d 8c .. 8c + 7
  v4f ks, vs;     // scales of keys 16t + 4g .. +3
};

// the 16-key group of quarter qr (from k0 + 16 qr, clamped into [lo, hi]), whose block
// is entry 0 .. 127 of the split
__device__ __forceinline__ XHalf xquarter(const DecodeArgs& a, const Split& sp, int k0, int qr) {
  XHalf r;
  r.hk0 = clampi(k0 + 16 * qr, sp.lo & ~15, sp.hi & ~15);
  const int local = clampi((r.hk0 >> a.pool.page_shift) - sp.first_block, 0, 127);
  const int page = local < 64 ? page_uniform(sp.tab, local) : page_uniform(sp.tab2, local - 64);
  r.ph = (int64_t)page * a.pool.num_kv_heads + sp.kvh;
  return r;
}
__device__ __forceinline__ void iload_k(IBuf& t, const DecodeArgs& a, const Split& sp, int k0) {
  constexpr int NC = 128 / 16;
  const int S = a.pool.page_size, c = sp.lane & 15, g = sp.lane >> 4;
#pragma unroll
  for (int qr = 0; qr < 4; ++qr) {
    const XHalf x = xquarter(a, sp, k0, qr);
    const uint4* kb = reinterpret_cast<const uint4*>(a.pool.k) + x.ph * NC * S + (x.hk0 & (S - 1)) + (g * S + c);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      t.k[qr][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)4 * s * S));
  }
}
__device__ __forceinline__ void iload_v(IBuf& t, const DecodeArgs& a, const Split& sp, int k0) {
  constexpr int D = 128;
  const int S = a.pool.page_size, c = sp.lane & 15, g = sp.lane >> 4;
#pragma unroll
  for (int qr = 0; qr < 4; ++qr) {
    const XHalf x = xquarter(a, sp, k0, qr);
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(a.pool.v) + (x.ph * S + (x.hk0 & (S - 1))) * D +
                              (4 * g * D + 8 * c);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vb + r * D));
      t.v[qr][r][0] = w[0];
      t.v[qr][r][1] = w[1];
    }
  }
}
__device__ __forceinline__ void iload_scales(IBuf& t, const DecodeArgs& a, const Split& sp, int k0, bool kside) {
  const int S = a.pool.page_size, sh = a.pool.page_shift, c = sp.lane & 15, g = sp.lane >> 4;
  const int g0 = clampi(k0 + 16 * (c >> 2) + 4 * g, sp.lo & ~3, sp.hi & ~3);
  const int local = clampi((g0 >> sh) - sp.first_block, 0, 127);
  const int p1 = page_of_lane(sp.tab, local & 63), p2 = page_of_lane(sp.tab2, local & 63);
  const int page = local < 64 ? p1 : p2;
  const int64_t si = ((int64_t)page * a.pool.num_kv_heads + sp.kvh) * S + (g0 & (S - 1));
  if (kside) t.ks = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.pool.k_scale + si));
  else t.vs = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.pool.v_scale + si));
}

// o[i] = byte i of s0, s1, s2, s3 (a 4 x 4 byte transpose)
__device__ __forceinline__ void transpose4x4(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3, uint32_t (&o)[4]) {
  const uint32_t u0 = __builtin_amdgcn_perm(s1, s0, 0x05010400u);  // s0.0 s1.0 s0.1 s1.1
  const uint32_t u1 = __builtin_amdgcn_perm(s1, s0, 0x07030602u);  // s0.2 s1.2 s0.3 s1.3
  const uint32_t u2 = __builtin_amdgcn_perm(s3, s2, 0x05010400u);
  const uint32_t u3 = __builtin_amdgcn_perm(s3, s2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(u2, u0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
}

// least E with |x| < 2^E (x != 0)
__device__ __forceinline__ int bound_exp(float x) { return __builtin_amdgcn_frexp_expf(x); }
// limb t (0..3) of the integer n = trunc(|y| 2^(27 - E)) < 2^27
__device__ __forceinline__ uint32_t limb_of(uint32_t n, int t) { return (n >> (21 - 7 * t)) & 127u; }

// Q of an item as the B operand of the int8 score product: for d step s, lane (c, g)
// holds limb t of head h's scaled query at d = 16(4s + g) + j, j = 0..15, as signed
// bytes, from qraw[16s + j] = Q[h][16(4s + g) + j].  Every wave finds the head's bound
// (the lanes (c, g) of one c hold all 128 d of the head between them) and returns the
// lane's score weight 2^(e_h - 6 - 7t); waves 0 and 1 store steps 0 and 1.
__device__ __forceinline__ float iqueries(const float (&qraw)[32], float qscale, int lane, int w, u32x4* qs) {
  const int t = (lane & 15) >> 2;
  float y[32], mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    y[i] = qraw[i] * qscale;
    mx = fmaxf(mx, fabsf(y[i]));
  }
  mx = wave_xor_max(mx, 16);
  mx = wave_xor_max(mx, 32);
  const int e = mx > 0.0f ? bound_exp(mx) : 0;  // a zero head has zero limbs
  if (w < 2) {
    uint32_t wd[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float v = w == 0 ? y[4 * qd + b] : y[16 + 4 * qd + b];
        const uint32_t c = limb_of((uint32_t)__builtin_ldexpf(fabsf(v), 27 - e), t);
        x |= ((v < 0.0f ? 0u - c : c) & 255u) << (8 * b);
      }
      wd[qd] = x;
    }
    qs[w * 64 + lane] = u32x4{wd[0], wd[1], wd[2], wd[3]};
  }
  return __builtin_ldexpf(1.0f, e - 6 - 7 * t);
}

// One 64-key tile on the operands in t; MORE: each part of t is reloaded with the next
// tile's (from k_next) once used (a compile-time choice: loads under a run-time
// condition made the compiler copy the loaded registers at the loop's end, which waits
// for every load in flight).  qs: the item's Q limb operands in LDS ([d step][lane]);
// wq: this lane's score weight; o: [d tile].  Lazy running max as in xtile.  l is this
// lane's part: the item's sum runs over the head's 16 lanes.
template <bool MORE, typename Hook = NoHook>
__device__ __forceinline__ void itile(const DecodeArgs& a, const Split& sp, IBuf& t, int k0, int k_next,
                                      const u32x4* qs, float wq, v4f (&o)[8], float& m, float& l,
                                      Hook hook = Hook()) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const int c = sp.lane & 15, g = sp.lane >> 4, term = c >> 2;
  const bool b0 = term & 1, b1 = term & 2;
  constexpr bool more = MORE;
  hook();  // (as in xtile4)
  // ---- V of this tile into B operand order (byte n of each key's 8 for d tile n =
  // 4hw + i), so the next tile's V loads can go out now
  uint32_t vt[2][4][4];  // [hw][quarter][i]
#pragma unroll
  for (int hw = 0; hw < 2; ++hw)
#pragma unroll
    for (int qr = 0; qr < 4; ++qr)
      transpose4x4(t.v[qr][0][hw], t.v[qr][1][hw], t.v[qr][2][hw], t.v[qr][3][hw], vt[hw][qr]);
  __builtin_amdgcn_sched_barrier(0);
  if (more) iload_v(t, a, sp, k_next);
  // ---- scores: limb sums of keys 16qr + 4g + r, weighted
  const i32x4 q0 = __builtin_bit_cast(i32x4, qs[sp.lane]), q1 = __builtin_bit_cast(i32x4, qs[64 + sp.lane]);
  float sw[4][4];
#pragma unroll
  for (int qr = 0; qr < 4; ++qr) {
    i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, t.k[qr][0]), q0, i32x4{0, 0, 0, 0},
                                                       0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, t.k[qr][1]), q1, acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) sw[qr][r] = (float)acc[r] * wq;
  }
  if (more) iload_k(t, a, sp, k_next);
  // reduce-scatter over limb lanes: with lane c ^ 4 keep the quarters of parity t % 2,
  // then with lane c ^ 8 keep quarter t
  float s4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float hv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float keep = b0 ? sw[2 * j + 1][r] : sw[2 * j][r];
      const float send = b0 ? sw[2 * j][r] : sw[2 * j + 1][r];
      hv[j] = keep + __shfl_xor(send, 4, 64);
    }
    const float keep = b1 ? hv[1] : hv[0], send = b1 ? hv[0] : hv[1];
    s4[r] = (keep + ror8f(send)) * t.ks[r];
  }
  if (more) iload_scales(t, a, sp, k_next, true);
  // ---- mask, online softmax for head h over the keys 16t + 4g + r
  float tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = k0 + 16 * term + 4 * g + r;
    s4[r] = (key >= sp.lo && key <= sp.k_end) ? s4[r] : -INFINITY;
    tmax = fmaxf(tmax, s4[r]);
  }
  tmax = wave_xor_max(tmax, 4);
  tmax = fmaxf(tmax, ror8f(tmax));
  tmax = wave_xor_max(tmax, 16);
  tmax = wave_xor_max(tmax, 32);
  const float m_new = (m == -INFINITY || tmax > m + 8.0f) ? tmax : m;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = (m == -INFINITY) ? 1.0f : fast_exp2(m - m_use);
  float psum = 0.0f, pmax = 0.0f, pv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = fast_exp2(s4[r] - m_use);
    psum += p;
    pv[r] = p > 0.0f ? p * t.vs[r] : 0.0f;
    pmax = fmaxf(pmax, pv[r]);
  }
  l = l * alpha + psum;
  m = m_new;
  if (more) iload_scales(t, a, sp, k_next, false);
  pmax = wave_xor_max(pmax, 4);
  pmax = fmaxf(pmax, ror8f(pmax));
  pmax = wave_xor_max(pmax, 16);
  pmax = wave_xor_max(pmax, 32);
  const int E = pmax > 0.0f ? bound_exp(pmax) : 0;
  // limbs of this lane's 4 keys: dw[u] = limb u of keys r = 0..3 (byte r), for lane u
  uint32_t n4[4], dw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) n4[r] = (uint32_t)__builtin_ldexpf(pv[r], 27 - E);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    dw[u] = limb_of(n4[0], u) | (limb_of(n4[1], u) << 8) | (limb_of(n4[2], u) << 16) | (limb_of(n4[3], u) << 24);
  // transpose over limb lanes: lane t ends with limb t of every quarter's keys
  uint32_t own[2], rcv[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // columns t % 2 + 2k: rows t and t ^ 1
    own[k] = b0 ? dw[1 + 2 * k] : dw[2 * k];
    const uint32_t send = b0 ? dw[2 * k] : dw[1 + 2 * k];
    rcv[k] = (uint32_t)__shfl_xor((int)send, 4, 64);
  }
  const uint32_t m_t = b1 ? own[1] : own[0], m_t1 = b1 ? rcv[1] : rcv[0];   // rows t, t ^ 1
  const uint32_t m_t2 = ror8(b1 ? own[0] : own[1]), m_t3 = ror8(b1 ? rcv[0] : rcv[1]);  // rows t ^ 2, t ^ 3
  uint32_t pw[4];
#pragma unroll
  for (int qr = 0; qr < 4; ++qr) {  // dword qr = row qr = row t ^ (qr ^ t)
    const bool x0 = ((qr & 1) != 0) != b0, x1 = ((qr & 2) != 0) != b1;
    pw[qr] = x1 ? (x0 ? m_t3 : m_t2) : (x0 ? m_t1 : m_t);
  }
  const i32x4 pa = i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
  // ---- rescale: accumulator row 4g + r belongs to head r; its limb g weighs 2^(E_r - 6 - 7g)
  if (__any(alpha != 1.0f)) {
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, r, 64);
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[n][r] *= ar[r];
  }
  float wv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) wv[r] = __builtin_ldexpf(1.0f, __builtin_amdgcn_readlane(E, r) - 6 - 7 * g);
  // ---- values
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int hw = n >> 2, i = n & 3;
    const i32x4 vb = i32x4{(int)vt[hw][0][i], (int)vt[hw][1][i], (int)vt[hw][2][i], (int)vt[hw][3][i]};
    const i32x4 r32 = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa, vb, i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) o[n][r] += (float)r32[r] * wv[r];
  }
}

// Waves per workgroup; they share one split, and the split's combine waits for the
// slowest of them.  Waves drift apart over a split (their loads are served at
// different rates), so the register-tile paths use 2 waves on half-size splits; the
// exact-split paths build their query operands one d step per wave, so they have 4.
template <bool XP> struct DecodeWaves { static constexpr int value = XP ? 4 : 2; };
// Workgroups per CU the register budget is sized for: 2 waves per SIMD (f32 tiles need
// twice the registers of the others, so the f32 register-tile kernel gets 1).
template <int KVT, bool XP> struct DecodeOcc {
  static constexpr int value = (KVT == KV_F32 && !XP) ? 1 : 2;
};
// Head groups per sequence: an item covers one KV head when G = 8 (both slots of a
// register tile hold its 8 query heads) or on the exact-split paths (one KV head per
// wave); the register tiles at G <= 4 hold two KV heads, one per slot.
template <int G, bool XP> struct OneKvHead { static constexpr bool value = G == 8 || XP; };

// ---------------------------------------------------------------- work items
// A work item is one split of one sequence for one head group.  Items are numbered
// densely, longest first: every sequence's whole splits, then the partial ones (a
// sequence's first split when the window cuts into it, its last when the length is
// not a multiple of the split size) in NBKT buckets of decreasing tile count.
// Workgroups are persistent and take items in that order (the first statically, then
// from a counter in the workspace), so the launch ends on its shortest items and
// no workgroup is spent on a split that does not exist.  Every workgroup rebuilds the
// numbering in LDS from the lengths (prefix sums over the batch).
constexpr int NBKT = 4;

struct SeqSplits { int lo, hi, s_first, s_last, f_first, f_last, nf, p0, p1, np; };  // partial splits p0, p1 (np of them)

template <bool RING>
__device__ __forceinline__ SeqSplits seq_splits(const DecodeArgs& a, int L) {
  SeqSplits r;
  const int sk = a.split_keys;
  if (!RING) L = min(L, a.max_blocks * a.pool.page_size);  // a ring has no end
  r.np = 0;
  r.p0 = r.p1 = 0;
  if (L <= 0) {
    r.lo = 0; r.hi = -1; r.s_first = 0; r.s_last = -1; r.f_first = 0; r.f_last = -1; r.nf = 0;
    return r;
  }
  r.hi = L - 1;
  r.lo = a.window > 0 ? max(0, L - a.window) : 0;
  r.s_first = r.lo / sk;
  r.s_last = r.hi / sk;
  r.f_first = (r.lo + sk - 1) / sk;  // first split wholly inside [lo, hi]
  r.f_last = (r.hi + 1) / sk - 1;    // last one
  r.nf = max(0, r.f_last - r.f_first + 1);
  // (no run-time array indexing here: such arrays would live in scratch memory)
  const bool first_partial = r.s_first < r.f_first || r.s_first > r.f_last;
  const bool last_partial = r.s_last != r.s_first && (r.s_last < r.f_first || r.s_last > r.f_last);
  r.np = (int)first_partial + (int)last_partial;
  r.p0 = first_partial ? r.s_first : r.s_last;
  r.p1 = r.s_last;
  return r;
}

// tiles of split s (its keys inside [lo, hi], from a 32-key boundary)
__device__ __forceinline__ int split_tiles(const DecodeArgs& a, const SeqSplits& ss, int s) {
  const int k_begin = max(s * a.split_keys, ss.lo) & ~(TK - 1);
  const int k_end = min((s + 1) * a.split_keys - 1, ss.hi);
  return (k_end - k_begin) / TK + 1;
}

__device__ __forceinline__ int tile_bucket(const DecodeArgs& a, int tiles) {
  const int per = a.split_keys / TK;
  return min(NBKT - 1, (tiles - 1) * NBKT / per);
}

// first index b in [0, n) with incl[b] > x (incl non-decreasing, incl[n-1] > x)
__device__ __forceinline__ int lds_upper(const int* incl, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// The LDS tables: per sequence its length and the inclusive prefix sums of its whole
// splits and of its partial splits in each bucket.
struct ItemTables {
  int* len;
  int* full;
  int* bkt[NBKT];
};
constexpr int TABLE_INTS = 2 + NBKT;  // ints of LDS per sequence

// Item number -> (sequence, head group, split).  Workgroup-uniform (made scalar).
struct Item { int b, y, split; };
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <bool RING>
__device__ __forceinline__ Item item_of_lds(const DecodeArgs& a, const ItemTables& t, int it, int gy);
template <bool RING>
__device__ __forceinline__ Item item_of(const DecodeArgs& a, const ItemTables& t, int it, int gy) {
  Item r = item_of_lds<RING>(a, t, uni(it), gy);
  r.b = uni(r.b); r.y = uni(r.y); r.split = uni(r.split);
  return r;
}
template <bool RING>
__device__ __forceinline__ Item item_of_lds(const DecodeArgs& a, const ItemTables& t, int it, int gy) {
  Item r;
  const int n = a.batch;
  int pair = it / gy;
  r.y = it - pair * gy;
  const int n_full = t.full[n - 1];
  if (pair < n_full) {
    r.b = lds_upper(t.full, n, pair);
    const SeqSplits ss = seq_splits<RING>(a, t.len[r.b]);
    r.split = ss.f_first + (pair - (t.full[r.b] - ss.nf));
    return r;
  }
  pair -= n_full;
  int k = NBKT - 1;
  for (; k > 0; --k) {  // buckets of longer splits first
    if (pair < t.bkt[k][n - 1]) break;
    pair -= t.bkt[k][n - 1];
  }
  r.b = lds_upper(t.bkt[k], n, pair);
  const SeqSplits ss = seq_splits<RING>(a, t.len[r.b]);
  const int before = t.bkt[k][r.b] - (r.b > 0 ? t.bkt[k][r.b - 1] : 0);  // this sequence's count in k
  const int local = pair - (t.bkt[k][r.b] - before);
  // the local-th of this sequence's partial splits that fall in bucket k
  const bool in0 = ss.np > 0 && tile_bucket(a, split_tiles(a, ss, ss.p0)) == k;
  r.split = (in0 && local == 0) ? ss.p0 : ss.p1;
  return r;
}

// Per-wave operands of an item that do not depend on its length: the block-table
// entries of the split (one per lane; a split spans at most 64 pages) and the raw
// queries.  They are only loaded here; the scale is applied when the item starts, so
// loads issued for the next item are not waited on before then.
template <int NQR>
struct ItemOps {
  int tab, tab2;  // (tab2: int8 tile only)
  float q[NQR];
};

// first q head of this lane's slot, and whether the lane's head exists
template <int G>
__device__ __forceinline__ void item_heads(const DecodeArgs& a, int y, int lane, int& qh_base, bool& head_on) {
  const int slot = lane >> 5, j = lane & 3;
  if constexpr (G == 8) {
    qh_base = y * 8 + slot * 4;
    head_on = true;
  } else {
    const int kvh = y * 2 + slot;
    qh_base = kvh * G;
    head_on = kvh < a.pool.num_kv_heads && (G >= 4 || j < G);
  }
}

// query registers per lane: register tiles D / 8, the bf16-split tiles 8 (one d step
// per wave), the int8 tile 32 (both d steps: every wave needs the head's bound)
template <int D, bool XP, bool XI> struct ItemQ { static constexpr int value = XI ? 32 : (XP ? 8 : D / 8); };

template <int D, int G, bool XP, bool XI, bool RING>
__device__ __forceinline__ void item_ops(const DecodeArgs& a, const Item& it, int lane, int w,
                                         ItemOps<ItemQ<D, XP, XI>::value>& op) {
  const int first_block = (it.split * a.split_keys) >> a.pool.page_shift;
  const int entry = RING ? (first_block + lane) % a.ring : min(first_block + lane, a.max_blocks - 1);
  op.tab = a.block_tables[(int64_t)it.b * a.max_blocks + entry];
  if constexpr (XI) {
    const int e2 = RING ? (first_block + 64 + lane) % a.ring : min(first_block + 64 + lane, a.max_blocks - 1);
    op.tab2 = a.block_tables[(int64_t)it.b * a.max_blocks + e2];
  }
  if constexpr (XI) {
    // lane (c, g): head c % 4 of the group, d = 16g .. 16g + 15 and 64 + 16g .. + 15
    const int c = lane & 15, g = lane >> 4;
    const float* qp = a.q + ((int64_t)it.b * a.num_q_heads + it.y * G + (c & (G - 1))) * D + 16 * g;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 x = *reinterpret_cast<const float4*>(qp + 64 * s + 4 * u);
        op.q[16 * s + 4 * u] = x.x; op.q[16 * s + 4 * u + 1] = x.y;
        op.q[16 * s + 4 * u + 2] = x.z; op.q[16 * s + 4 * u + 3] = x.w;
      }
  } else if constexpr (XP) {
    // lane (c, g) of wave w: head c % G of the group, d = 32g + 8w .. +7 (step w)
    const int c = lane & 15, g = lane >> 4;
    const float* qp = a.q + ((int64_t)it.b * a.num_q_heads + it.y * G + (c & (G - 1))) * D + 32 * g + 8 * w;
    const float4 x0 = *reinterpret_cast<const float4*>(qp);
    const float4 x1 = *reinterpret_cast<const float4*>(qp + 4);
    op.q[0] = x0.x; op.q[1] = x0.y; op.q[2] = x0.z; op.q[3] = x0.w;
    op.q[4] = x1.x; op.q[5] = x1.y; op.q[6] = x1.z; op.q[7] = x1.w;
  } else {
    int qh_base;
    bool head_on;
    item_heads<G>(a, it.y, lane, qh_base, head_on);
    // register t of lane (slot, kg, j) holds Q[head j][d = 8t + kg], read from a valid
    // head whatever the lane (an absent head is zeroed by its scale)
    const int kg = (lane >> 2) & 7, j = lane & 3;
    const int hq = min(qh_base + j, a.num_q_heads - 1);
    const float* qp = a.q + ((int64_t)it.b * a.num_q_heads + hq) * D + kg;
#pragma unroll
    for (int t = 0; t < D / 8; ++t) op.q[t] = qp[8 * t];
  }
}

// Partial states cross workgroups (and XCDs, whose L2 caches are not coherent with
// each other) inside one launch when the splits merge in place.  They are then
// written and read with device-scope relaxed atomics, which go to the coherent level
// instead of a non-coherent cached copy; the writer waits for its stores to complete
// before it counts its split, and the reader loads only after it has seen the count.
// No cache-wide writeback or invalidate is needed (device-scope fences would cost
// one on every split).
template <bool COH>
__device__ __forceinline__ void store1(float* p, float v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ void store2(float* p, float x, float y) {
  if constexpr (!COH) {
    *reinterpret_cast<float2*>(p) = make_float2(x, y);
    return;
  }
  const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool COH>
__device__ __forceinline__ float2 load2(const float* p) {
  if constexpr (!COH) return *reinterpret_cast<const float2*>(p);
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Merge of the splits s_base .. s_base + ns - 1 of q heads hq0 .. hq0 + nh - 1 of
// sequence b (nh <= 8) by one workgroup of NTHR threads, from partial states that
// other workgroups of the same launch stored: m* = max m_s, then
// o = sum 2^(m_s - m*) acc_s / sum 2^(m_s - m*) l_s (log2 units), the sums taken in
// split order.  Thread t takes head t / (NTHR / 8) and VPT consecutive values of it;
// up to MB splits are loaded in one batch, so a sequence of at most MB splits waits
// for one round of loads.
template <int D, int NTHR>
__device__ __forceinline__ void merge_group(const DecodeArgs& a, int b, int hq0, int nh, int s_base, int ns, int tid) {
  constexpr int TPH = NTHR / 8, VPT = D / TPH, NP = VPT / 2, MB = 16;
  static_assert(VPT == 2 || VPT == 4 || VPT == 8, "values per thread");
  const int h = tid / TPH, d0 = (tid % TPH) * VPT;
  if (h >= nh) return;
  const int64_t bh = (int64_t)b * a.num_q_heads + hq0 + h;
  const float* ml = a.ws_ml + (bh * a.n_split + s_base) * 2;
  const float* acc = a.ws_acc + (bh * a.n_split + s_base) * D + d0;
  float o[VPT] = {};
  float l = 0.0f, mstar = -INFINITY;
  auto add = [&](float wgt, const float2 (&v)[NP]) {
#pragma unroll
    for (int n = 0; n < NP; ++n) { o[2 * n] += wgt * v[n].x; o[2 * n + 1] += wgt * v[n].y; }
  };
  for (int s0 = 0; s0 < ns; s0 += MB) {  // m* first (one pass when ns <= MB: the loads are shared)
    if (ns <= MB) break;
    float2 x[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) x[u] = load2<true>(ml + 2 * min(s0 + u, ns - 1));
#pragma unroll
    for (int u = 0; u < MB; ++u)
      if (s0 + u < ns) mstar = fmaxf(mstar, x[u].x);
  }
  for (int s0 = 0; s0 < ns; s0 += MB) {
    float2 x[MB], av[MB][NP];
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int sx = min(s0 + u, ns - 1);
      x[u] = load2<true>(ml + 2 * sx);
#pragma unroll
      for (int n = 0; n < NP; ++n) av[u][n] = load2<true>(acc + (int64_t)sx * D + 2 * n);
    }
    if (ns <= MB) {
#pragma unroll
      for (int u = 0; u < MB; ++u)
        if (u < ns) mstar = fmaxf(mstar, x[u].x);
    }
    const float mu = mstar == -INFINITY ? 0.0f : mstar;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      if (s0 + u < ns) {
        const float wgt = fast_exp2(x[u].x - mu);
        l += wgt * x[u].y;
        add(wgt, av[u]);
      }
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* dst = a.out + bh * D + d0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) dst[i] = l > 0.0f ? o[i] * inv : 0.0f;
}

// The workgroup that finishes last resets the item and finished-workgroup counters
// for the next call.  A workgroup's last claim has returned before it arrives here, so
// no claim can follow the reset.
__device__ __forceinline__ void workgroup_done(const DecodeArgs& a, int tid) {
  if (tid == 0) {
    if (atomicAdd(a.ws_ctrl + 1, 1) == (int)gridDim.x - 1) {
      __hip_atomic_store(a.ws_ctrl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ws_ctrl + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Persistent workgroups of NWD waves.  For each claimed item, wave w takes the
// split's tiles w, w + NWD, ... with its own softmax state; the NWD states are then
// combined through LDS in wave order, so the result depends on the split alone, not
// on which workgroup ran it or when.  The next item number is claimed during wave
// 0's last tile of the current item (so an item goes to a workgroup only when that
// workgroup is nearly free: longest-processing-time-first scheduling), and the next
// item's table entries and queries load while the current item is combined.
template <int KVT, int D, int G, bool XP, bool RING>
__global__ __launch_bounds__(64 * DecodeWaves<XP>::value, (DecodeOcc<KVT, XP>::value)) void decode_split_kernel(
    DecodeArgs a) {
  constexpr int NWD = DecodeWaves<XP>::value;
  constexpr int NTHR = 64 * NWD;
  using GE = Geo<KVT, D>;
  constexpr int NT = GE::NT;
  constexpr int PF = DecodePrefetch<KVT, D, G>::value;
  // the int8 tile (exact-split path, int8 codes) takes 64 keys per wave, the others 32
  constexpr bool XI = XP && KVT == KV_INT8;
  constexpr int TKW = XI ? 64 : TK;
  constexpr int STEP = NWD * TKW;
  constexpr int NQR = ItemQ<D, XP, XI>::value;
  // In-place merge on the exact-split path only (measured: it saves the merge launch
  // there, while the register-tile kernels lose more than that to it)
  constexpr bool FUSE = XP;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = lane >> 5, kg = (lane >> 2) & 7, j = lane & 3;
  const int H = a.pool.num_kv_heads;
  const int gy = OneKvHead<G, XP>::value ? H : (H + 1) / 2;

  extern __shared__ int dyn[];  // [TABLE_INTS][batch]
  ItemTables tabs;
  tabs.len = dyn;
  tabs.full = dyn + a.batch;
#pragma unroll
  for (int k = 0; k < NBKT; ++k) tabs.bkt[k] = dyn + (2 + k) * a.batch;
  __shared__ int c_carry[1 + NBKT], c_wsum[NWD][1 + NBKT], s_claim[1], s_last[1];
  __shared__ float c_acc[NWD][NT * 4][64];    // [wave][value i*4 + r][lane]
  __shared__ float c_m[NWD][8], c_l[NWD][8];  // [wave][slot*4 + head]
  __shared__ bf16x8 x_q[XP ? 8 * 64 : 1];  // exact-split path: Q3 operands of the item

  // ---- numbering tables (inclusive block scans over the batch, NTHR at a time)
  if (tid <= NBKT) c_carry[tid] = 0;
  __syncthreads();
  for (int c0 = 0; c0 < a.batch; c0 += NTHR) {
    const int b = c0 + tid;
    int cnt[1 + NBKT];
#pragma unroll
    for (int k = 0; k <= NBKT; ++k) cnt[k] = 0;
    if (b < a.batch) {
      const int L = a.seq_lens[b];
      const SeqSplits ss = seq_splits<RING>(a, L);
      cnt[0] = ss.nf;
      const int b0 = ss.np > 0 ? tile_bucket(a, split_tiles(a, ss, ss.p0)) : -1;
      const int b1 = ss.np > 1 ? tile_bucket(a, split_tiles(a, ss, ss.p1)) : -1;
#pragma unroll
      for (int k = 0; k < NBKT; ++k) cnt[1 + k] = (int)(b0 == k) + (int)(b1 == k);
      tabs.len[b] = L;
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
      for (int k = 0; k <= NBKT; ++k) {
        const int x = __shfl_up(cnt[k], d, 64);
        if (lane >= d) cnt[k] += x;
      }
    }
    if (lane == 63) {
#pragma unroll
      for (int k = 0; k <= NBKT; ++k) c_wsum[w][k] = cnt[k];
    }
    __syncthreads();
    int base[1 + NBKT];
#pragma unroll
    for (int k = 0; k <= NBKT; ++k) {
      base[k] = c_carry[k];
      for (int u = 0; u < w; ++u) base[k] += c_wsum[u][k];
    }
    if (b < a.batch) {
      tabs.full[b] = base[0] + cnt[0];
#pragma unroll
      for (int k = 0; k < NBKT; ++k) tabs.bkt[k][b] = base[1 + k] + cnt[1 + k];
    }
    __syncthreads();
    if (tid == NTHR - 1) {
#pragma unroll
      for (int k = 0; k <= NBKT; ++k) c_carry[k] = base[k] + cnt[k];
    }
    __syncthreads();
  }
  int n_pairs = tabs.full[a.batch - 1];
#pragma unroll
  for (int k = 0; k < NBKT; ++k) n_pairs += tabs.bkt[k][a.batch - 1];
  const int n_items = uni(n_pairs * gy);
  if (FUSE && a.fuse_merge) {
    // rows of empty sequences are zero (they have no items); workgroup i takes
    // sequences i, i + n_wg, ...
    for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
      if (tabs.len[b] > 0) continue;
      float* o = a.out + (int64_t)b * a.num_q_heads * D;
      for (int i = tid; i < a.num_q_heads * D; i += NTHR) o[i] = 0.0f;
    }
  }
  // the first item of each workgroup is fixed; later ones come from the counter
  const int n_wg = gridDim.x;
  int cur = blockIdx.x;
  if (cur >= n_items) {  // workgroup-uniform
    if constexpr (FUSE) workgroup_done(a, tid);
    return;
  }
  Item it = item_of<RING>(a, tabs, cur, gy);
  ItemOps<NQR> op;
  item_ops<D, G, XP, XI, RING>(a, it, lane, w, op);
  float wq = 0.0f;  // int8 tile: this lane's score weight for the item
  if constexpr (XP) {  // scores come out in log2 units
    if constexpr (XI) wq = iqueries(op.q, a.qscale, lane, w, reinterpret_cast<u32x4*>(x_q));
    else if constexpr (G == 4) xqueries4(op.q, a.qscale, lane, w, x_q);
    else xqueries(op.q, a.qscale, lane, w, x_q);
  }

  // In-place merge.  A split's partial states are counted one item later, when the
  // workgroup's next item reaches its combine: by then the coherent stores have long
  // completed, so the wait before the count costs nothing.  The workgroup whose count
  // completes a (sequence, head group) merges it.  pend_b < 0: nothing to count.
  int pend_b = -1, pend_y = 0, pend_ns = 0, pend_base = 0;
  auto count_pending = [&]() {  // after a barrier that follows every wave's wait
    int* arrive = a.ws_arrive + (int64_t)pend_b * gy + pend_y;
    if (tid == 0) s_last[0] = atomicAdd(arrive, 1) == pend_ns - 1;
    __syncthreads();
    if (s_last[0]) {
      int hq0, nh;
      if constexpr (OneKvHead<G, XP>::value) {
        hq0 = pend_y * G; nh = G;
      } else {
        hq0 = pend_y * 2 * G; nh = (pend_y * 2 + 1 < H) ? 2 * G : G;
      }
      merge_group<D, NTHR>(a, pend_b, hq0, nh, pend_base, pend_ns, tid);
      if (tid == 0) __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
    }
    pend_b = -1;
  };

  for (;;) {
    __syncthreads();  // the previous item's combine is done everywhere
    int claimed = 0;
    // The next item is claimed during wave 0's last tile of this one (at its start on
    // the register and G = 4 tiles, at its end on the G = 8 tile), so items go to
    // workgroups in the order they become free (longest first).  The count is read
    // only at the combine, so the add's round trip overlaps the rest of that tile.
    auto claim = [&]() { if (tid == 0) claimed = atomicAdd(a.ws_ctrl, 1); };

    // ---- this item
    int kvh, qh_base;
    bool slot_on;
    if constexpr (G == 8) {
      kvh = it.y; qh_base = kvh * 8 + slot * 4; slot_on = true;
    } else if constexpr (XP) {  // G = 4: the wave's 4 heads are the first slot's
      kvh = it.y; qh_base = kvh * 4; slot_on = slot == 0;
    } else {
      kvh = it.y * 2 + slot; slot_on = kvh < H; qh_base = kvh * G;
      if (!slot_on) kvh = H - 1;  // keep addresses valid; results are discarded
    }
    float q[XP ? 1 : D / 8];
    if constexpr (!XP) {
      int qb;
      bool head_on;
      item_heads<G>(a, it.y, lane, qb, head_on);
      const float qs = head_on ? a.qscale : 0.0f;  // scores come out in log2 units
#pragma unroll
      for (int t = 0; t < D / 8; ++t) q[t] = op.q[t] * qs;
    }
    const SeqSplits ss = seq_splits<RING>(a, uni(tabs.len[it.b]));
    const int k_begin = max(it.split * a.split_keys, ss.lo) & ~(TK - 1);
    const int k_end = min((it.split + 1) * a.split_keys - 1, ss.hi);  // inclusive
    Split sp;
    sp.kvh = kvh; sp.lo = ss.lo; sp.hi = ss.hi; sp.k_end = k_end; sp.lane = lane;
    sp.first_block = (it.split * a.split_keys) >> a.pool.page_shift;
    sp.tab = clampi(op.tab, 0, a.pool.num_pages - 1);
    sp.tab2 = XI ? clampi(op.tab2, 0, a.pool.num_pages - 1) : 0;

    float m = -INFINITY, l = 0.0f;
    int k0 = k_begin + w * TKW;
    if constexpr (XP && G == 4) {
      float zero;  // (made inside the item loop, as below)
      asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
      v4f ox[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) ox[n] = v4f{zero, zero, zero, zero};
      static_assert(KVT == KV_BF16 || KVT == KV_INT8, "the G = 4 exact-split tiles take bf16 or int8 K and V");
      if constexpr (XI) {
        const u32x4* qi = reinterpret_cast<const u32x4*>(x_q);
        IBuf ib;
        k0 = uni(k0);  // (wave-uniform: the page lookups stay scalar)
        if (k0 <= k_end) {
          iload_k(ib, a, sp, k0);
          iload_scales(ib, a, sp, k0, true);
          iload_scales(ib, a, sp, k0, false);
          iload_v(ib, a, sp, k0);
          while (k0 + STEP <= k_end) {
            itile<true>(a, sp, ib, k0, k0 + STEP, qi, wq, ox, m, l);
            k0 += STEP;
          }
          itile<false>(a, sp, ib, k0, k0 + STEP, qi, wq, ox, m, l, claim);
        } else {
          claim();
        }
      } else {
        X4Buf xb;
        if (k0 <= k_end) {
          x4load_k(xb, a, sp, k0);
          x4load_v(xb, a, sp, k0);
          while (k0 + STEP <= k_end) {
            xtile4(a, sp, xb, k0, k0 + STEP, x_q, ox, m, l);
            k0 += STEP;
          }
          xtile4(a, sp, xb, k0, k0 + STEP, x_q, ox, m, l, claim);
        } else {
          claim();
        }
      }
      // ---- l and O summed over the lane groups (rows 4g + r: term g of head r); lane
      // group 0 writes d tiles 0-3, group 1 d tiles 4-7 of head r, d = 8c + n, to LDS
      // (value (d / 32) * 4 + r, column d % 32).  (On the int8 tile the lanes of a head
      // also hold different keys.)
      if constexpr (XI) {
        l = wave_xor_sum(l, 4);
        l += ror8f(l);
      }
      l = wave_xor_sum(l, 16);
      l = wave_xor_sum(l, 32);
      const int c = lane & 15, g = lane >> 4;
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = ox[n][r] + __shfl_xor(ox[n][r], 16, 64);
          v += __shfl_xor(v, 32, 64);
          if (g == (n >> 2)) {
            const int d = 8 * c + n;
            c_acc[w][(d >> 5) * 4 + r][d & 31] = v;
          }
        }
      if (lane < 4) { c_m[w][lane] = m; c_l[w][lane] = l; }
    } else if constexpr (XP) {
      static_assert(kv_fp8(KVT) && G == 8, "the G = 8 exact-split tile takes fp8 codes");
      // accumulators start from a zero made inside the item loop, so the compiler
      // does not keep 64 zero registers live (or spilled) across it
      float zero;
      asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
      v4f ox[2][8];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int n = 0; n < 8; ++n) ox[t][n] = v4f{zero, zero, zero, zero};
      const bf16x8* qsw = x_q;
      XBuf xb;
      if (k0 <= k_end) {
        constexpr bool SC = kv_scaled(KVT);
        xload<SC>(xb, a, sp, k0);
        while (k0 + STEP <= k_end) {
          xtile<SC>(a, sp, xb, k0, k0 + STEP, qsw, ox, m, l);
          k0 += STEP;
        }
        xtile<SC>(a, sp, xb, k0, k0 + STEP, qsw, ox, m, l, claim);
      } else {
        claim();
      }
      // ---- l over the lane groups; O = hi rows + mid rows (lanes + 32) + lo rows; to LDS
      l = wave_xor_sum(l, 16);
      l = wave_xor_sum(l, 32);
      const int c = lane & 15, g = lane >> 4;
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = (ox[0][n][r] + __shfl_xor(ox[0][n][r], 32, 64)) + ox[1][n][r];
          if (g < 2) {
            const int d = 8 * c + n;  // head 4g + r
            c_acc[w][(d & 3) * 4 + r][g * 32 + (d >> 2)] = v;
          }
        }
      if (lane < 8) { c_m[w][lane] = m; c_l[w][lane] = l; }
    } else {
      v4f o[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) o[i] = v4f{0, 0, 0, 0};
      // K of the wave's next tile is prefetched into the other buffer where registers
      // allow it; otherwise each tile loads its own K.  The wave's last tile is peeled
      // so the next item's operands load with it.
      KBuf<KVT, D> kA, kB;
      VBuf<KVT, D> vA, vB_;
      VBuf<KVT, D>& vB = (PF >= 2) ? vB_ : vA;  // one V buffer unless V is prefetched
      int par = 0;
      if constexpr (PF == 0) {
        // no buffer alternates: one copy of the tile in the loop, one peeled
        if (k0 <= k_end) {
          while (k0 + STEP <= k_end) {
            decode_tile<KVT, D, PF>(a, sp, kA, kB, vA, vB, k0, k0 + STEP, q, o, m, l);
            k0 += STEP;
          }
          decode_tile<KVT, D, PF>(a, sp, kA, kB, vA, vB, k0, k0 + STEP, q, o, m, l, claim);
        } else {
          claim();
        }
      } else if (k0 <= k_end) {
        if constexpr (PF >= 1) load_k<KVT, D>(kA, a, sp, k0);
        if constexpr (PF >= 2) load_v<KVT, D>(vA, a, sp, k0);
        while (k0 + STEP <= k_end) {
          decode_tile<KVT, D, PF>(a, sp, kA, kB, vA, vB, k0, k0 + STEP, q, o, m, l);
          k0 += STEP;
          if (k0 + STEP > k_end) { par = 1; break; }
          decode_tile<KVT, D, PF>(a, sp, kB, kA, vB, vA, k0, k0 + STEP, q, o, m, l);
          k0 += STEP;
        }
        if (par) {  // the last tile's prefetched operands sit in the B buffers
          kA = kB;
          if constexpr (PF >= 2) vA = vB;
        }
        decode_tile<KVT, D, PF>(a, sp, kA, kB, vA, vB, k0, k0 + STEP, q, o, m, l, claim);
      } else {
        claim();
      }
      // ---- l per head summed over the slot's key groups; the wave's state to LDS
      l = wave_xor_sum(l, 4);
      l = wave_xor_sum(l, 8);
      l = wave_xor_sum(l, 16);
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) c_acc[w][i * 4 + r][lane] = o[i][r];
      if (kg == 0) { c_m[w][slot * 4 + j] = m; c_l[w][slot * 4 + j] = l; }
    }
    if (FUSE && pend_b >= 0) __builtin_amdgcn_s_waitcnt(0);  // the previous item's partial stores have completed
    if (tid == 0) s_claim[0] = n_wg + claimed;
    __syncthreads();
    // the next item's table entries and queries load while this one is combined
    // (a claim is n_wg + a counter that starts at zero; any other value, from a
    // workspace whose counter was not zero, ends the workgroup rather than indexing
    // outside the tables)
    const int nxt = uni(s_claim[0]);
    const bool has_next = nxt >= n_wg && nxt < n_items;
    Item nit = it;
    ItemOps<NQR> nop;
    if (has_next) {
      nit = item_of<RING>(a, tabs, nxt, gy);
      item_ops<D, G, XP, XI, RING>(a, nit, lane, w, nop);
    }
    if constexpr (FUSE) {
      if (pend_b >= 0) count_pending();
    }

    // ---- combine in wave order: value v = i*4 + r of this lane is head slot*4 + r,
    // d = (lane % 32) * NT + i, except on the G = 4 exact-split tile, where
    // d = 32 i + lane % 32: there 32 lanes store a whole 128-byte line of a partial
    // state at once (coherent stores write through to memory, and a line stored in
    // pieces is written as several).  (On the G = 8 tile the same layout cost spilled
    // registers; it keeps the first.)  Wave w finishes the values v with v % NWD == w.
    const bool single = (ss.s_first == ss.s_last);
    const int d_base = (lane & 31) * NT;
#pragma unroll
    for (int v = 0; v < NT * 4; ++v) {
      if (v % NWD != w) continue;
      const int i = v >> 2, r = v & 3;
      if (!slot_on || (G < 4 && r >= G)) continue;
      const int h = slot * 4 + r;
      float ms = -INFINITY;
#pragma unroll
      for (int u = 0; u < NWD; ++u) ms = fmaxf(ms, c_m[u][h]);
      const float mu = (ms == -INFINITY) ? 0.0f : ms;
      float lsum = 0.0f, acc = 0.0f;
#pragma unroll
      for (int u = 0; u < NWD; ++u) {
        const float wt = fast_exp2(c_m[u][h] - mu);
        lsum += wt * c_l[u][h];
        acc += wt * c_acc[u][v][lane];
      }
      const int hq = qh_base + r, d = (XP && G == 4) ? 32 * i + (lane & 31) : d_base + i;
      if (single) {
        a.out[((int64_t)it.b * a.num_q_heads + hq) * D + d] = lsum > 0.0f ? acc * (1.0f / lsum) : 0.0f;
      } else {
        // a ring row's splits are stored from its first (their numbers grow without end)
        const int rs = RING ? it.split - ss.s_first : it.split;
        store1<FUSE>(a.ws_acc + (((int64_t)it.b * a.num_q_heads + hq) * a.n_split + rs) * D + d, acc);
        if (i == 0 && (lane & 31) == 0)
          store2<FUSE>(a.ws_ml + (((int64_t)it.b * a.num_q_heads + hq) * a.n_split + rs) * 2, ms, lsum);
      }
    }
    if (FUSE && !single && a.fuse_merge) {
      pend_b = it.b; pend_y = it.y; pend_ns = ss.s_last - ss.s_first + 1; pend_base = RING ? 0 : ss.s_first;
    }
    if (!has_next) break;  // workgroup-uniform
    // (exact-split path: every wave is past the barrier above, so no tile reads the
    // query operands any more; the loop-top barrier publishes the new ones)
    if constexpr (XP) {
      if constexpr (XI) wq = iqueries(nop.q, a.qscale, lane, w, reinterpret_cast<u32x4*>(x_q));
      else if constexpr (G == 4) xqueries4(nop.q, a.qscale, lane, w, x_q);
      else xqueries(nop.q, a.qscale, lane, w, x_q);
    }
    it = nit;
    op = nop;
  }
  if constexpr (FUSE) {
    if (pend_b >= 0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      count_pending();
    }
    workgroup_done(a, tid);
  }
}

// Combine the splits of each (sequence, q head): m* = max m_s,
// o = sum 2^(m_s - m*) acc_s / sum 2^(m_s - m*) l_s (log2 units).  Sequences with one
// split were finished by the split kernel; empty sequences get zeros.  Lane s holds
// split s's (m, l) (64 splits per pass), so the max and the sum over splits are wave
// reductions; the accumulators are read eight splits per batch of loads.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.num_q_heads;
  const int lane = threadIdx.x;
  constexpr int PER = D / 64;
  if (bh == 0 && lane == 0) a.ws_ctrl[0] = 0;  // item counter, for the next call
  float* dst = a.out + (int64_t)bh * D + lane * PER;
  const int L = a.ring > 0 ? a.seq_lens[b] : min(a.seq_lens[b], a.max_blocks * a.pool.page_size);
  if (L <= 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) dst[i] = 0.0f;
    return;
  }
  const int hi = L - 1;
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int s0 = lo / a.split_keys, s1 = hi / a.split_keys;
  if (s0 == s1) return;
  const int ns = s1 - s0 + 1;
  const int base = a.ring > 0 ? 0 : s0;  // ring rows store their splits from the first
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + (int64_t)bh * a.n_split + base;
  const float* acc = a.ws_acc + ((int64_t)bh * a.n_split + base) * D + lane * PER;
  if (ns <= 16) {
    // every load at once (one round of latency), then the same sums in the same order
    const float2 x = lane < ns ? ml[lane] : make_float2(-INFINITY, 0.0f);
    float av[16][PER];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int s = min(u, ns - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) av[u][i] = acc[(int64_t)s * D + i];
    }
    float mx = x.x;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = wave_xor_max(mx, m);
    if (mx == -INFINITY) mx = 0.0f;
    const float w = lane < ns ? fast_exp2(x.x - mx) : 0.0f;
    float ls = w * x.y;
    float o[PER] = {};
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u < ns) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += wu * av[u][i];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ls = wave_xor_sum(ls, m);
    const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) dst[i] = ls > 0.0f ? o[i] * inv : 0.0f;
    return;
  }
  float mstar = -INFINITY;
  for (int c = lane; c < ns; c += 64) mstar = fmaxf(mstar, ml[c].x);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mstar = wave_xor_max(mstar, m);
  if (mstar == -INFINITY) mstar = 0.0f;
  float o[PER] = {};
  float l = 0.0f;
  for (int c = 0; c < ns; c += 64) {
    float w = 0.0f;
    if (c + lane < ns) {
      const float2 x = ml[c + lane];
      w = fast_exp2(x.x - mstar);
      l += w * x.y;
    }
    const int n = min(64, ns - c);
    for (int u0 = 0; u0 < n; u0 += 8) {
      float av[8][PER];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = c + min(u0 + u, n - 1);
#pragma unroll
        for (int i = 0; i < PER; ++i) av[u][i] = acc[(int64_t)s * D + i];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = (u0 + u < n) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u0 + u)) : 0.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += wu * av[u][i];
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) l = wave_xor_sum(l, m);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[i] = l > 0.0f ? o[i] * inv : 0.0f;
}

// Resident workgroups of one kernel instantiation at a given dynamic LDS size on the
// current device, cached per (instantiation, device): each instantiation has its own
// register and LDS footprint, and devices may differ in CU count.
constexpr int RW_DEVICES = 64;
template <auto kernel>
int resident_workgroups(int threads, size_t dyn_lds) {
  static std::mutex mu;
  static int cached[RW_DEVICES];
  static size_t cached_lds[RW_DEVICES];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= RW_DEVICES) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0 || cached_lds[dev] != dyn_lds) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn_lds) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = per_cu * cus;
    cached_lds[dev] = dyn_lds;
  }
  return cached[dev];
}

template <int KVT, int D, int G, bool XP, bool RING>
hipError_t decode_launch_split_r(const DecodeArgs& a, hipStream_t s) {
  const int H = a.pool.num_kv_heads;
  const int64_t gy = OneKvHead<G, XP>::value ? H : (H + 1) / 2;
  const size_t dyn = (size_t)TABLE_INTS * a.batch * sizeof(int);
  const int64_t upper = (int64_t)a.batch * a.n_split * gy;
  constexpr int threads = 64 * DecodeWaves<XP>::value;
  const int64_t wgs = std::min<int64_t>(upper, resident_workgroups<decode_split_kernel<KVT, D, G, XP, RING>>(threads, dyn));
  DecodeArgs c = a;
  // in place on the exact-split path when the arrival counters cover every head group
  c.fuse_merge = XP && gy <= DECODE_ARRIVE_GROUPS;
  hipLaunchKernelGGL((decode_split_kernel<KVT, D, G, XP, RING>), dim3((unsigned)wgs), dim3(threads), dyn, s, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.fuse_merge) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(a.batch * a.num_q_heads)), dim3(64), 0, s, c);
  return hipGetLastError();
}

// ring tables take their own instantiations, so the full-table kernels carry none of
// the ring's extra live values
template <int KVT, int D, int G, bool XP>
hipError_t decode_launch_split_x(const DecodeArgs& a, hipStream_t s) {
  return a.ring > 0 ? decode_launch_split_r<KVT, D, G, XP, true>(a, s) : decode_launch_split_r<KVT, D, G, XP, false>(a, s);
}

template <int KVT, int D, int G>
hipError_t decode_launch_split(const DecodeArgs& a, hipStream_t s) {
  // the exact-split tiles serve fp8 pools at D = 128, G = 8, and bf16 and int8 pools at
  // D = 128, G = 4, with pages of >= 16 (a 16-key group never straddles a page)
  if constexpr ((kv_fp8(KVT) && D == 128 && G == 8) || ((KVT == KV_BF16 || KVT == KV_INT8) && D == 128 && G == 4)) {
    if (a.pool.page_size >= 16) return decode_launch_split_x<KVT, D, G, true>(a, s);
  }
  return decode_launch_split_x<KVT, D, G, false>(a, s);
}

template <int KVT, int D>
hipError_t decode_dispatch_g(const DecodeArgs& a, hipStream_t s) {
  hipError_t e;
  switch (a.group) {
    case 8: e = decode_launch_split<KVT, D, 8>(a, s); break;
    case 4: e = decode_launch_split<KVT, D, 4>(a, s); break;
    case 2: e = decode_launch_split<KVT, D, 2>(a, s); break;
    default: e = decode_launch_split<KVT, D, 1>(a, s); break;
  }
  return e;
}

template <int KVT>
hipError_t decode_dispatch(const DecodeArgs& a, hipStream_t s) {
  if (a.pool.head_dim == 128) return decode_dispatch_g<KVT, 128>(a, s);
  return decode_dispatch_g<KVT, 64>(a, s);
}

}  // namespace

// Keys per split (measured on the c2, c2r, c2i and c5 layers): 4,096 for fp8 pools,
// 1,024 for bf16 pools on the G = 4 exact-split tile, 2,048 for int8 pools on the
// int8 tile (as many bytes per item as the bf16 tile's), 512 for the register tiles.
// A split's table entries sit one per lane, so it spans at most 64 pages (128 on the
// int8 tile, two per lane).
int decode_split_keys(int kv_dtype, int group, int head_dim, int page_size) {
  const bool x4 = (kv_dtype == KV_BF16 || kv_dtype == KV_INT8) && group == 4 && head_dim == 128 && page_size >= 16;
  const bool xi = x4 && kv_dtype == KV_INT8;
  const int want = kv_fp8(kv_dtype) ? 4096 : (xi ? 2048 : (x4 ? 1024 : 512));
  const int most = (xi ? 128 : 64) * page_size;
  return want < most ? want : most;
}

// Batches larger than DECODE_BATCH_CHUNK run as consecutive launches over slices of
// the batch (the per-workgroup item tables hold 24 bytes of LDS per sequence).
// Sequences are independent, so a slice computes exactly what the whole batch would.
// The exact-split kernel merges its splits in place when the arrival counters cover
// every head group; otherwise a merge kernel follows the split kernel.

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t s) {
  for (int b0 = 0; b0 < a.batch; b0 += DECODE_BATCH_CHUNK) {
    DecodeArgs c = a;
    c.batch = std::min(DECODE_BATCH_CHUNK, a.batch - b0);
    c.q = a.q + (int64_t)b0 * a.num_q_heads * a.pool.head_dim;
    c.out = a.out + (int64_t)b0 * a.num_q_heads * a.pool.head_dim;
    c.block_tables = a.block_tables + (int64_t)b0 * a.max_blocks;
    c.seq_lens = a.seq_lens + b0;
    hipError_t e;
    switch (kv_dtype) {
      case KV_F32: e = decode_dispatch<KV_F32>(c, s); break;
      case KV_BF16: e = decode_dispatch<KV_BF16>(c, s); break;
      case KV_FP8: e = decode_dispatch<KV_FP8>(c, s); break;
      case KV_FP8U: e = decode_dispatch<KV_FP8U>(c, s); break;
      default: e = decode_dispatch<KV_INT8>(c, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tl
