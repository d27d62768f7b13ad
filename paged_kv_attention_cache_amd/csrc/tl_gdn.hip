// GATED_DELTA_RULE, decode step: the Gated DeltaNet recurrence over a pool of f32
// recurrent states indexed by state slot ("How serving works in Tlaloc",
// "Linear-attention layers: the state pools").  Per sequence b and head h, with S the
// [128][128] state of slot[b] (key index i, value index j):
//   S = S * exp(g);  u = k^T S;  S += k (outer) beta (v - u);  o = q^T S.
// A row at position 0 starts from zero state; slot -1 is a pad (no state touched,
// output row 0).
//
// One workgroup of 256 threads per (sequence, head): thread (half, j) holds rows
// 64*half .. +63 of column j in registers, so the state is read once and written once
// (HBM-bound: 128 KiB per (sequence, head)); the two reductions over i are a lane-local
// sum of 64 terms and one LDS exchange between the halves, in a fixed order.
#include "tl_internal.h"

namespace tl {
namespace {

constexpr int GD = 128;   // key and value dimension of a head
constexpr int GWG = 256;  // threads: 2 halves of the key rows x 128 value columns

__global__ __launch_bounds__(GWG) void gdn_decode_kernel(GdnArgs a) {
  __shared__ float s_k[GD], s_q[GD], s_red[2][GD];
  const int bh = blockIdx.x;
  const int b = bh / a.num_heads, h = bh - b * a.num_heads;
  const int t = threadIdx.x, j = t & (GD - 1), half = t >> 7;
  const int64_t row = (int64_t)b * a.num_heads + h;
  const int slot = a.slots[b];
  if (slot < 0 || slot >= a.num_slots) {  // a pad (or a slot outside the pool): output 0
    if (half == 0) a.out[row * GD + j] = 0.0f;
    return;
  }
  const bool fresh = a.positions[b] == 0;
  if (half == 0) s_k[j] = a.k[row * GD + j];
  else s_q[j] = a.q[row * GD + j];
  float* S = a.pool + ((int64_t)slot * a.num_heads + h) * GD * GD + (int64_t)(64 * half) * GD + j;
  float s[64];
  if (fresh) {
#pragma unroll
    for (int r = 0; r < 64; ++r) s[r] = 0.0f;
  } else {
#pragma unroll
    for (int r = 0; r < 64; ++r) s[r] = __builtin_nontemporal_load(S + r * GD);
  }
  const float decay = fast_exp2(a.g[row] * LOG2E);
  const float beta = a.beta[row];
  const float vj = a.v[row * GD + j];
  __syncthreads();
  // u_j = sum_i k_i S[i][j] after the decay
  float u = 0.0f;
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    s[r] *= decay;
    u += s_k[64 * half + r] * s[r];
  }
  s_red[half][j] = u;
  __syncthreads();
  u = s_red[0][j] + s_red[1][j];
  const float delta = beta * (vj - u);
  // S += k (outer) delta;  o_j = sum_i q_i S[i][j]
  float o = 0.0f;
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    s[r] += s_k[64 * half + r] * delta;
    o += s_q[64 * half + r] * s[r];
  }
  __syncthreads();  // both halves have read u from s_red
  s_red[half][j] = o;
#pragma unroll
  for (int r = 0; r < 64; ++r) __builtin_nontemporal_store(s[r], S + r * GD);
  __syncthreads();
  if (half == 0) a.out[row * GD + j] = s_red[0][j] + s_red[1][j];
}

}  // namespace

hipError_t launch_gdn_decode(const GdnArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(gdn_decode_kernel, dim3((unsigned)(a.batch * a.num_heads)), dim3(GWG), 0, s, a);
  return hipGetLastError();
}

}  // namespace tl
