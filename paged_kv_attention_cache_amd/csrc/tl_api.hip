// C ABI of libtl: argument validation on the host, then kernel launches on the
// caller's stream.  No allocation, no synchronisation (except the opt-in
// TL_VALIDATE=1 range checks, which copy index arrays to the host).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "tl_internal.h"

// The decode workspace of tl_paged_attn_decode_static, for callers that cannot
// allocate: one copy on every device the library runs on, held until the process
// ends.  Host code never uses this name as an address (on the host it is only a
// stand-in for the symbol); the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[TL_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_err[2048] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return TL_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

bool validate_mode() {
  const char* e = getenv("TL_VALIDATE");
  return e && e[0] == '1';
}

int check_pool(const char* fn, const tl_kv_pool* pool) {
  if (!pool) return fail(TL_ERR_INVALID, "%s: pool is NULL", fn);
  if (pool->dtype < TL_KV_F32 || pool->dtype > TL_KV_INT8)
    return fail(TL_ERR_UNSUPPORTED, "%s: pool->dtype (%d) is not a tl_kv_dtype", fn, pool->dtype);
  if (!pool->k) return fail(TL_ERR_INVALID, "%s: pool->k is NULL", fn);
  if (!pool->v) return fail(TL_ERR_INVALID, "%s: pool->v is NULL", fn);
  if (!aligned(pool->k, 16)) return fail(TL_ERR_INVALID, "%s: pool->k is not 16-byte aligned", fn);
  if (!aligned(pool->v, 16)) return fail(TL_ERR_INVALID, "%s: pool->v is not 16-byte aligned", fn);
  if (pool->dtype == TL_KV_FP8_E4M3 || pool->dtype == TL_KV_INT8) {
    if (!pool->k_scale) return fail(TL_ERR_INVALID, "%s: pool->k_scale is NULL for a scaled fp8 pool", fn);
    if (!pool->v_scale) return fail(TL_ERR_INVALID, "%s: pool->v_scale is NULL for a scaled fp8 pool", fn);
    if (!aligned(pool->k_scale, 16)) return fail(TL_ERR_INVALID, "%s: pool->k_scale is not 16-byte aligned", fn);
    if (!aligned(pool->v_scale, 16)) return fail(TL_ERR_INVALID, "%s: pool->v_scale is not 16-byte aligned", fn);
  }
  if (pool->num_pages <= 0) return fail(TL_ERR_INVALID, "%s: pool->num_pages (%d) must be > 0", fn, pool->num_pages);
  if (pool->num_kv_heads <= 0)
    return fail(TL_ERR_INVALID, "%s: pool->num_kv_heads (%d) must be > 0", fn, pool->num_kv_heads);
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(TL_ERR_UNSUPPORTED, "%s: pool->head_dim (%d) must be 64 or 128", fn, pool->head_dim);
  if (!is_pow2(pool->page_size) || pool->page_size < 8 || pool->page_size > 1024)
    return fail(TL_ERR_UNSUPPORTED, "%s: pool->page_size (%d) must be a power of two in [8, 1024]", fn,
                pool->page_size);
  if ((int64_t)pool->num_pages * pool->page_size >= ((int64_t)1 << 31))
    return fail(TL_ERR_UNSUPPORTED, "%s: pool->num_pages * pool->page_size must be < 2^31", fn);
  return TL_OK;
}

tl::PoolArgs pool_args(const tl_kv_pool* p) {
  tl::PoolArgs a;
  a.k = p->k; a.v = p->v; a.k_scale = p->k_scale; a.v_scale = p->v_scale;
  a.num_pages = p->num_pages; a.page_size = p->page_size; a.page_shift = log2i(p->page_size);
  a.num_kv_heads = p->num_kv_heads; a.head_dim = p->head_dim;
  return a;
}

int hip_fail(const char* fn, hipError_t e) {
  return fail(TL_ERR_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
}

template <typename T>
int copy_to_host(const char* fn, const char* what, const T* src, size_t n, std::vector<T>& dst, hipStream_t s) {
  dst.resize(n);
  if (n == 0) return TL_OK;
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(TL_ERR_HIP, "%s: TL_VALIDATE copy of %s failed (%s)", fn, what, hipGetErrorString(e));
  return TL_OK;
}

int check_tables(const char* fn, const tl_kv_pool* pool, const std::vector<int32_t>& tables, int32_t max_blocks,
                 int32_t b, int64_t positions_needed) {
  const int64_t blocks = (positions_needed + pool->page_size - 1) / pool->page_size;
  for (int64_t i = 0; i < blocks; ++i) {
    const int32_t p = tables[(size_t)b * max_blocks + i];
    if (p < 0 || p >= pool->num_pages)
      return fail(TL_ERR_INVALID, "%s: block_tables[%d][%lld] = %d is not a page of the pool (TL_VALIDATE)", fn, b,
                  (long long)i, p);
  }
  return TL_OK;
}

int check_group(const char* fn, const tl_kv_pool* pool, int32_t num_q_heads) {
  if (num_q_heads <= 0) return fail(TL_ERR_INVALID, "%s: num_q_heads (%d) must be > 0", fn, num_q_heads);
  if (num_q_heads % pool->num_kv_heads != 0)
    return fail(TL_ERR_INVALID, "%s: num_q_heads (%d) is not a multiple of pool->num_kv_heads (%d)", fn, num_q_heads,
                pool->num_kv_heads);
  const int g = num_q_heads / pool->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(TL_ERR_UNSUPPORTED, "%s: num_q_heads / num_kv_heads (%d) must be 1, 2, 4 or 8", fn, g);
  return TL_OK;
}

int64_t decode_nsplit(const tl_kv_pool* pool, int32_t num_q_heads, int32_t max_blocks) {
  const int sk = tl::decode_split_keys(pool->dtype, num_q_heads / pool->num_kv_heads, pool->head_dim, pool->page_size);
  const int64_t keys = (int64_t)max_blocks * pool->page_size;
  return (keys + sk - 1) / sk;
}

// Keys a ring row can score: the window, at most the ring's N = R * S slots.
int32_t ring_window(const tl_kv_pool* pool, int32_t ring_pages, int32_t window) {
  const int64_t n = (int64_t)ring_pages * pool->page_size;
  return (int32_t)(window > 0 ? std::min<int64_t>(window, n) : n);
}

// Splits a row of a ring touches: its keys are the last ring_window() positions,
// which span at most (w - 1) / sk + 2 splits of sk keys.
int64_t ring_nsplit(const tl_kv_pool* pool, int32_t num_q_heads, int32_t ring_pages, int32_t window) {
  const int sk = tl::decode_split_keys(pool->dtype, num_q_heads / pool->num_kv_heads, pool->head_dim, pool->page_size);
  return (ring_window(pool, ring_pages, window) - 1) / sk + 2;
}

size_t decode_ws_bytes(const tl_kv_pool* pool, int32_t batch, int32_t num_q_heads, int64_t ns) {
  // the control words and arrival counters (the same bytes whatever the shape), then
  // the partial states (acc, then m and l)
  return (size_t)tl::DECODE_WS_HEADER + (size_t)batch * num_q_heads * ns * (pool->head_dim + 2) * sizeof(float);
}

// Shared by the full-table and ring decode entries.  ring = 0: block_tables has
// max_blocks entries per row, block j at entry j; ring = R: R entries, block j at j % R.
int decode_common(const char* fn, const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                  const int32_t* block_tables, int32_t max_blocks, int32_t ring, const int32_t* seq_lens,
                  int32_t batch, int32_t window, float scale, float* out, void* workspace, size_t workspace_bytes,
                  void* stream) {
  int rc = check_pool(fn, pool);
  if (rc) return rc;
  if ((rc = check_group(fn, pool, num_q_heads))) return rc;
  if (batch < 0) return fail(TL_ERR_INVALID, "%s: batch (%d) must be >= 0", fn, batch);
  if (batch > 65535) return fail(TL_ERR_UNSUPPORTED, "%s: batch (%d) must be <= 65535", fn, batch);
  if (ring == 0) {
    if (max_blocks <= 0) return fail(TL_ERR_INVALID, "%s: max_blocks (%d) must be > 0", fn, max_blocks);
    if ((int64_t)max_blocks * pool->page_size >= ((int64_t)1 << 31))
      return fail(TL_ERR_UNSUPPORTED, "%s: max_blocks * page_size must be < 2^31", fn);
  } else {
    if (ring <= 0) return fail(TL_ERR_INVALID, "%s: ring_pages (%d) must be > 0", fn, ring);
    if ((int64_t)ring * pool->page_size >= ((int64_t)1 << 30))
      return fail(TL_ERR_UNSUPPORTED, "%s: ring_pages * page_size must be < 2^30", fn);
  }
  if (batch == 0) return ok();
  if (!q) return fail(TL_ERR_INVALID, "%s: q is NULL", fn);
  if (!out) return fail(TL_ERR_INVALID, "%s: out is NULL", fn);
  if (!block_tables) return fail(TL_ERR_INVALID, "%s: %s is NULL", fn, ring ? "ring_tables" : "block_tables");
  if (!seq_lens) return fail(TL_ERR_INVALID, "%s: seq_lens is NULL", fn);
  if (!aligned(q, 16)) return fail(TL_ERR_INVALID, "%s: q is not 16-byte aligned", fn);
  if (!aligned(out, 16)) return fail(TL_ERR_INVALID, "%s: out is not 16-byte aligned", fn);
  if (!aligned(block_tables, 4))
    return fail(TL_ERR_INVALID, "%s: %s is not 4-byte aligned", fn, ring ? "ring_tables" : "block_tables");
  if (!aligned(seq_lens, 4)) return fail(TL_ERR_INVALID, "%s: seq_lens is not 4-byte aligned", fn);
  const int64_t ns = ring ? ring_nsplit(pool, num_q_heads, ring, window) : decode_nsplit(pool, num_q_heads, max_blocks);
  const size_t need = decode_ws_bytes(pool, batch, num_q_heads, ns);
  if (!workspace || workspace_bytes < need)
    return fail(TL_ERR_WORKSPACE, "%s: workspace (%zu bytes) is smaller than the %zu bytes required", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if (!aligned(workspace, 16)) return fail(TL_ERR_INVALID, "%s: workspace is not 16-byte aligned", fn);
  hipStream_t s = (hipStream_t)stream;
  const int32_t width = ring ? ring : max_blocks;
  if (validate_mode()) {
    std::vector<int32_t> lens, tables;
    if ((rc = copy_to_host(fn, "seq_lens", seq_lens, (size_t)batch, lens, s))) return rc;
    if ((rc = copy_to_host(fn, "block_tables", block_tables, (size_t)batch * width, tables, s))) return rc;
    const int64_t n_ring = (int64_t)ring * pool->page_size;
    for (int32_t b = 0; b < batch; ++b) {
      if (lens[b] < 0 || (!ring && (int64_t)lens[b] > (int64_t)max_blocks * pool->page_size))
        return fail(TL_ERR_INVALID, "%s: seq_lens[%d] = %d is outside [0, max_blocks * page_size] (TL_VALIDATE)", fn,
                    b, lens[b]);
      const int64_t used = ring ? std::min<int64_t>(lens[b], n_ring) : lens[b];
      if ((rc = check_tables(fn, pool, tables, width, b, used))) return rc;
    }
  }
  tl::DecodeArgs a;
  a.pool = pool_args(pool);
  a.q = q; a.block_tables = block_tables; a.seq_lens = seq_lens; a.out = out;
  a.ws_ctrl = reinterpret_cast<int*>(workspace);  // same place for every shape
  a.ws_arrive = reinterpret_cast<int*>(static_cast<char*>(workspace) + 16);
  a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + tl::DECODE_WS_HEADER);
  a.ws_ml = a.ws_acc + (size_t)batch * num_q_heads * ns * pool->head_dim;
  a.num_q_heads = num_q_heads; a.group = num_q_heads / pool->num_kv_heads; a.max_blocks = width;
  a.batch = batch; a.window = ring ? ring_window(pool, ring, window) : window;
  a.ring = ring;
  a.split_keys = tl::decode_split_keys(pool->dtype, a.group, pool->head_dim, pool->page_size);
  a.n_split = (int)ns;
  a.fuse_merge = 0;  // chosen per kernel at launch
  a.qscale = scale * tl::LOG2E;
  hipError_t e = tl::launch_decode(a, pool->dtype, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int prefill_common(const char* fn, const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                   const int32_t* block_tables, int32_t max_blocks, int32_t ring, const int32_t* positions,
                   int32_t batch, int32_t tokens_per_row, int32_t window, float scale, float* out, void* stream) {
  int rc = check_pool(fn, pool);
  if (rc) return rc;
  if ((rc = check_group(fn, pool, num_q_heads))) return rc;
  if (batch < 0) return fail(TL_ERR_INVALID, "%s: batch (%d) must be >= 0", fn, batch);
  if (batch > 65535) return fail(TL_ERR_UNSUPPORTED, "%s: batch (%d) must be <= 65535", fn, batch);
  if (tokens_per_row < 0) return fail(TL_ERR_INVALID, "%s: tokens_per_row (%d) must be >= 0", fn, tokens_per_row);
  if (ring == 0) {
    if (max_blocks <= 0) return fail(TL_ERR_INVALID, "%s: max_blocks (%d) must be > 0", fn, max_blocks);
    if ((int64_t)max_blocks * pool->page_size >= ((int64_t)1 << 31))
      return fail(TL_ERR_UNSUPPORTED, "%s: max_blocks * page_size must be < 2^31", fn);
  } else {
    if (ring <= 0) return fail(TL_ERR_INVALID, "%s: ring_pages (%d) must be > 0", fn, ring);
    if ((int64_t)ring * pool->page_size >= ((int64_t)1 << 30))
      return fail(TL_ERR_UNSUPPORTED, "%s: ring_pages * page_size must be < 2^30", fn);
  }
  if ((int64_t)batch * tokens_per_row * num_q_heads >= ((int64_t)1 << 31) / 128)
    return fail(TL_ERR_UNSUPPORTED, "%s: batch * tokens_per_row * num_q_heads is too large for one call", fn);
  if (batch == 0 || tokens_per_row == 0) return ok();
  if (!q) return fail(TL_ERR_INVALID, "%s: q is NULL", fn);
  if (!out) return fail(TL_ERR_INVALID, "%s: out is NULL", fn);
  if (!block_tables) return fail(TL_ERR_INVALID, "%s: %s is NULL", fn, ring ? "ring_tables" : "block_tables");
  if (!positions) return fail(TL_ERR_INVALID, "%s: positions is NULL", fn);
  if (!aligned(q, 16)) return fail(TL_ERR_INVALID, "%s: q is not 16-byte aligned", fn);
  if (!aligned(out, 16)) return fail(TL_ERR_INVALID, "%s: out is not 16-byte aligned", fn);
  if (!aligned(block_tables, 4))
    return fail(TL_ERR_INVALID, "%s: %s is not 4-byte aligned", fn, ring ? "ring_tables" : "block_tables");
  if (!aligned(positions, 4)) return fail(TL_ERR_INVALID, "%s: positions is not 4-byte aligned", fn);
  hipStream_t s = (hipStream_t)stream;
  const int32_t width = ring ? ring : max_blocks;
  if (validate_mode()) {
    std::vector<int32_t> pos, tables;
    if ((rc = copy_to_host(fn, "positions", positions, (size_t)batch * tokens_per_row, pos, s))) return rc;
    if ((rc = copy_to_host(fn, "block_tables", block_tables, (size_t)batch * width, tables, s))) return rc;
    const int64_t n_ring = (int64_t)ring * pool->page_size;
    for (int32_t b = 0; b < batch; ++b) {
      int64_t pmax = -1;
      for (int32_t t = 0; t < tokens_per_row; ++t) {
        const int32_t p = pos[(size_t)b * tokens_per_row + t];
        if (p < -1 || (!ring && (int64_t)p >= (int64_t)max_blocks * pool->page_size))
          return fail(TL_ERR_INVALID, "%s: positions[%d][%d] = %d is outside [-1, max_blocks * page_size) (TL_VALIDATE)",
                      fn, b, t, p);
        pmax = std::max<int64_t>(pmax, p);
      }
      const int64_t used = ring ? std::min<int64_t>(pmax + 1, n_ring) : pmax + 1;
      if ((rc = check_tables(fn, pool, tables, width, b, used))) return rc;
    }
  }
  tl::PrefillArgs a;
  a.pool = pool_args(pool);
  a.q = q; a.block_tables = block_tables; a.positions = positions; a.out = out;
  a.num_q_heads = num_q_heads; a.group = num_q_heads / pool->num_kv_heads; a.max_blocks = width;
  a.batch = batch; a.tokens_per_row = tokens_per_row;
  a.window = ring ? ring_window(pool, ring, window) : window;
  a.ring = ring;
  a.tokens_per_wg = tl::prefill_tokens_per_wg(a.group);
  a.n_qtiles = (tokens_per_row + a.tokens_per_wg - 1) / a.tokens_per_wg;
  a.qscale = scale * tl::LOG2E;
  hipError_t e = tl::launch_prefill(a, pool->dtype, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

// ------------------------------------------------- static scratch (no allocation)
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES];  // device address of `scratch` on each device, once set up

__global__ __launch_bounds__(256) void zero_words_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// This device's scratch address.  On the first call on a device (with that device
// current) the address is resolved with hipGetSymbolAddress and the workspace header
// is cleared by a fill kernel on `s`, ordered before the caller's kernels on that
// stream.  Later calls leave the header at zero themselves.
int static_scratch(const char* fn, hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(TL_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices the library tracks", fn, dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(fn, e);
    if (!p) return fail(TL_ERR_HIP, "%s: hipGetSymbolAddress gave no address for the static scratch", fn);
    const int words = (int)(tl::DECODE_WS_HEADER / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, static_cast<int*>(p),
                       words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(fn, e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TL_OK;
}

}  // namespace

namespace tl {
int set_error(int code, const char* msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return code;
}
}  // namespace tl

extern "C" {

const char* tl_last_error(void) { return g_err; }

int tl_abi_version(void) { return 1; }

int tl_kv_cache_write(const tl_kv_pool* pool, const float* k_new, const float* v_new, const int32_t* slots,
                      int64_t n_tokens, void* stream) {
  const char* fn = "tl_kv_cache_write";
  int rc = check_pool(fn, pool);
  if (rc) return rc;
  if (n_tokens < 0) return fail(TL_ERR_INVALID, "%s: n_tokens (%lld) must be >= 0", fn, (long long)n_tokens);
  if (n_tokens == 0) return ok();
  if (!k_new) return fail(TL_ERR_INVALID, "%s: k_new is NULL", fn);
  if (!v_new) return fail(TL_ERR_INVALID, "%s: v_new is NULL", fn);
  if (!slots) return fail(TL_ERR_INVALID, "%s: slots is NULL", fn);
  if (!aligned(k_new, 16)) return fail(TL_ERR_INVALID, "%s: k_new is not 16-byte aligned", fn);
  if (!aligned(v_new, 16)) return fail(TL_ERR_INVALID, "%s: v_new is not 16-byte aligned", fn);
  if (!aligned(slots, 4)) return fail(TL_ERR_INVALID, "%s: slots is not 4-byte aligned", fn);
  if (n_tokens * pool->num_kv_heads >= ((int64_t)1 << 31) / 8)
    return fail(TL_ERR_UNSUPPORTED, "%s: n_tokens * num_kv_heads is too large for one call", fn);
  hipStream_t s = (hipStream_t)stream;
  if (validate_mode()) {
    std::vector<int32_t> h;
    if ((rc = copy_to_host(fn, "slots", slots, (size_t)n_tokens, h, s))) return rc;
    const int64_t limit = (int64_t)pool->num_pages * pool->page_size;
    std::vector<int32_t> live;
    for (int64_t i = 0; i < n_tokens; ++i) {
      if (h[i] == -1) continue;
      if (h[i] < 0 || h[i] >= limit)
        return fail(TL_ERR_INVALID, "%s: slots[%lld] = %d is outside the pool (TL_VALIDATE)", fn, (long long)i, h[i]);
      live.push_back(h[i]);
    }
    std::sort(live.begin(), live.end());
    for (size_t i = 1; i < live.size(); ++i)
      if (live[i] == live[i - 1]) return fail(TL_ERR_INVALID, "%s: slot %d appears twice (TL_VALIDATE)", fn, live[i]);
  }
  tl::WriteArgs a;
  a.pool = pool_args(pool);
  a.k = pool->k; a.v = pool->v; a.k_scale = pool->k_scale; a.v_scale = pool->v_scale;
  a.k_new = k_new; a.v_new = v_new; a.slots = slots; a.n_tokens = n_tokens;
  hipError_t e = tl::launch_write(a, pool->dtype, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

size_t tl_paged_attn_decode_workspace_size(const tl_kv_pool* pool, int32_t batch, int32_t num_q_heads,
                                           int32_t max_blocks) {
  const char* fn = "tl_paged_attn_decode_workspace_size";
  if (check_pool(fn, pool) || check_group(fn, pool, num_q_heads)) return 0;
  if (batch <= 0 || max_blocks <= 0) return 0;
  return decode_ws_bytes(pool, batch, num_q_heads, decode_nsplit(pool, num_q_heads, max_blocks));
}

int tl_paged_attn_decode(const tl_kv_pool* pool, const float* q, int32_t num_q_heads, const int32_t* block_tables,
                         int32_t max_blocks, const int32_t* seq_lens, int32_t batch, int32_t window, float scale,
                         float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common("tl_paged_attn_decode", pool, q, num_q_heads, block_tables, max_blocks, 0, seq_lens, batch,
                       window, scale, out, workspace, workspace_bytes, stream);
}

int tl_paged_attn_decode_static(const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                                const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens, int32_t batch,
                                int32_t window, float scale, float* out, void* stream) {
  const char* fn = "tl_paged_attn_decode_static";
  int rc = check_pool(fn, pool);
  if (rc) return rc;
  if ((rc = check_group(fn, pool, num_q_heads))) return rc;
  if (batch < 0) return fail(TL_ERR_INVALID, "%s: batch (%d) must be >= 0", fn, batch);
  if (max_blocks <= 0) return fail(TL_ERR_INVALID, "%s: max_blocks (%d) must be > 0", fn, max_blocks);
  if ((int64_t)max_blocks * pool->page_size >= ((int64_t)1 << 31))
    return fail(TL_ERR_UNSUPPORTED, "%s: max_blocks * page_size must be < 2^31", fn);
  if (batch == 0) return ok();
  const size_t need = decode_ws_bytes(pool, batch, num_q_heads, decode_nsplit(pool, num_q_heads, max_blocks));
  if (need > (size_t)TL_STATIC_SCRATCH_BYTES)
    return fail(TL_ERR_WORKSPACE,
                "%s: this call needs %zu bytes of workspace, more than the %zu bytes of static scratch per device "
                "(pass a workspace to tl_paged_attn_decode instead)",
                fn, need, (size_t)TL_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = static_scratch(fn, (hipStream_t)stream, &ws))) return rc;
  return decode_common(fn, pool, q, num_q_heads, block_tables, max_blocks, 0, seq_lens, batch, window, scale, out, ws,
                       (size_t)TL_STATIC_SCRATCH_BYTES, stream);
}

size_t tl_paged_attn_decode_ring_workspace_size(const tl_kv_pool* pool, int32_t batch, int32_t num_q_heads,
                                                int32_t ring_pages, int32_t window) {
  const char* fn = "tl_paged_attn_decode_ring_workspace_size";
  if (check_pool(fn, pool) || check_group(fn, pool, num_q_heads)) return 0;
  if (batch <= 0 || ring_pages <= 0 || (int64_t)ring_pages * pool->page_size >= ((int64_t)1 << 30)) return 0;
  return decode_ws_bytes(pool, batch, num_q_heads, ring_nsplit(pool, num_q_heads, ring_pages, window));
}

int tl_paged_attn_decode_ring(const tl_kv_pool* pool, const float* q, int32_t num_q_heads, const int32_t* ring_tables,
                              int32_t ring_pages, const int32_t* seq_lens, int32_t batch, int32_t window, float scale,
                              float* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tl_paged_attn_decode_ring";
  if (ring_pages <= 0) return fail(TL_ERR_INVALID, "%s: ring_pages (%d) must be > 0", fn, ring_pages);
  return decode_common(fn, pool, q, num_q_heads, ring_tables, ring_pages, ring_pages, seq_lens, batch, window, scale,
                       out, workspace, workspace_bytes, stream);
}

size_t tl_paged_attn_prefill_workspace_size(const tl_kv_pool* pool, int32_t batch, int32_t tokens_per_row,
                                            int32_t num_q_heads, int32_t max_blocks) {
  (void)pool; (void)batch; (void)tokens_per_row; (void)num_q_heads; (void)max_blocks;
  return 0;
}

int tl_paged_attn_prefill(const tl_kv_pool* pool, const float* q, int32_t num_q_heads, const int32_t* block_tables,
                          int32_t max_blocks, const int32_t* positions, int32_t batch, int32_t tokens_per_row,
                          int32_t window, float scale, float* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  (void)workspace; (void)workspace_bytes;
  return prefill_common("tl_paged_attn_prefill", pool, q, num_q_heads, block_tables, max_blocks, 0, positions, batch,
                        tokens_per_row, window, scale, out, stream);
}

int tl_paged_attn_prefill_ring(const tl_kv_pool* pool, const float* q, int32_t num_q_heads, const int32_t* ring_tables,
                               int32_t ring_pages, const int32_t* positions, int32_t batch, int32_t tokens_per_row,
                               int32_t window, float scale, float* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const char* fn = "tl_paged_attn_prefill_ring";
  (void)workspace; (void)workspace_bytes;
  if (ring_pages <= 0) return fail(TL_ERR_INVALID, "%s: ring_pages (%d) must be > 0", fn, ring_pages);
  return prefill_common(fn, pool, q, num_q_heads, ring_tables, ring_pages, ring_pages, positions, batch,
                        tokens_per_row, window, scale, out, stream);
}

int tl_gated_delta_rule_decode(float* state_pool, int32_t num_slots, int32_t num_heads, int32_t head_dim,
                               const float* q, const float* k, const float* v, const float* g, const float* beta,
                               const int32_t* state_slots, const int32_t* positions, int32_t batch, float* out,
                               void* stream) {
  const char* fn = "tl_gated_delta_rule_decode";
  if (head_dim != 128) return fail(TL_ERR_UNSUPPORTED, "%s: head_dim (%d) must be 128", fn, head_dim);
  if (num_heads <= 0) return fail(TL_ERR_INVALID, "%s: num_heads (%d) must be > 0", fn, num_heads);
  if (num_slots <= 0) return fail(TL_ERR_INVALID, "%s: num_slots (%d) must be > 0", fn, num_slots);
  if ((int64_t)num_slots * num_heads >= ((int64_t)1 << 31) / (128 * 128))
    return fail(TL_ERR_UNSUPPORTED, "%s: num_slots * num_heads is too large", fn);
  if (batch < 0) return fail(TL_ERR_INVALID, "%s: batch (%d) must be >= 0", fn, batch);
  if ((int64_t)batch * num_heads >= ((int64_t)1 << 31) / 128)
    return fail(TL_ERR_UNSUPPORTED, "%s: batch * num_heads is too large for one call", fn);
  if (batch == 0) return ok();
  const void* ptrs[] = {state_pool, q, k, v, g, beta, state_slots, positions, out};
  const char* names[] = {"state_pool", "q", "k", "v", "g", "beta", "state_slots", "positions", "out"};
  for (int i = 0; i < 9; ++i) {
    if (!ptrs[i]) return fail(TL_ERR_INVALID, "%s: %s is NULL", fn, names[i]);
    if (!aligned(ptrs[i], (i < 4 || i == 8) ? 16 : 4))
      return fail(TL_ERR_INVALID, "%s: %s is not %d-byte aligned", fn, names[i], (i < 4 || i == 8) ? 16 : 4);
  }
  hipStream_t s = (hipStream_t)stream;
  int rc;
  if (validate_mode()) {
    std::vector<int32_t> sl;
    if ((rc = copy_to_host(fn, "state_slots", state_slots, (size_t)batch, sl, s))) return rc;
    std::vector<int32_t> used;
    for (int32_t b = 0; b < batch; ++b) {
      if (sl[b] == -1) continue;
      if (sl[b] < 0 || sl[b] >= num_slots)
        return fail(TL_ERR_INVALID, "%s: state_slots[%d] = %d is outside the pool (TL_VALIDATE)", fn, b, sl[b]);
      used.push_back(sl[b]);
    }
    std::sort(used.begin(), used.end());
    for (size_t i = 1; i < used.size(); ++i)
      if (used[i] == used[i - 1]) return fail(TL_ERR_INVALID, "%s: state slot %d appears twice (TL_VALIDATE)", fn, used[i]);
  }
  tl::GdnArgs a;
  a.pool = state_pool; a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.slots = state_slots; a.positions = positions; a.out = out;
  a.batch = batch; a.num_heads = num_heads; a.num_slots = num_slots;
  hipError_t e = tl::launch_gdn_decode(a, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int tl_kv_copy_pages(const tl_kv_pool* pool, const int32_t* src_pages, const int32_t* dst_pages, int32_t n,
                     void* stream) {
  const char* fn = "tl_kv_copy_pages";
  int rc = check_pool(fn, pool);
  if (rc) return rc;
  if (n < 0) return fail(TL_ERR_INVALID, "%s: n (%d) must be >= 0", fn, n);
  if (n == 0) return ok();
  if (n > 65535) return fail(TL_ERR_UNSUPPORTED, "%s: n (%d) must be <= 65535", fn, n);
  if (!src_pages || !dst_pages) return fail(TL_ERR_INVALID, "%s: src_pages/dst_pages is NULL", fn);
  if (!aligned(src_pages, 4) || !aligned(dst_pages, 4))
    return fail(TL_ERR_INVALID, "%s: src_pages/dst_pages is not 4-byte aligned", fn);
  tl::CopyPagesArgs a;
  const int bytes = pool->dtype == TL_KV_F32 ? 4 : pool->dtype == TL_KV_BF16 ? 2 : 1;
  const bool scaled = pool->dtype == TL_KV_FP8_E4M3 || pool->dtype == TL_KV_INT8;
  a.k = pool->k; a.v = pool->v;
  a.k_scale = scaled ? pool->k_scale : nullptr; a.v_scale = scaled ? pool->v_scale : nullptr;
  a.num_pages = pool->num_pages;
  a.units = (int64_t)pool->num_kv_heads * pool->page_size * pool->head_dim * bytes / 16;
  a.scales = (int64_t)pool->num_kv_heads * pool->page_size;
  hipError_t e = tl::launch_copy_pages(a, src_pages, dst_pages, n, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int tl_slot_mapping(const int32_t* tables, int32_t width, int32_t ring_pages, const int32_t* positions,
                    int32_t batch, int32_t tokens_per_row, int32_t page_size, int32_t num_pages, int32_t* slots,
                    void* stream) {
  const char* fn = "tl_slot_mapping";
  if (batch < 0) return fail(TL_ERR_INVALID, "%s: batch (%d) must be >= 0", fn, batch);
  if (tokens_per_row < 0) return fail(TL_ERR_INVALID, "%s: tokens_per_row (%d) must be >= 0", fn, tokens_per_row);
  if (width <= 0) return fail(TL_ERR_INVALID, "%s: width (%d) must be > 0", fn, width);
  if (ring_pages < 0 || ring_pages > width)
    return fail(TL_ERR_INVALID, "%s: ring_pages (%d) must be in [0, width = %d]", fn, ring_pages, width);
  if (!is_pow2(page_size) || page_size < 8 || page_size > 1024)
    return fail(TL_ERR_UNSUPPORTED, "%s: page_size (%d) must be a power of two in [8, 1024]", fn, page_size);
  if (num_pages <= 0) return fail(TL_ERR_INVALID, "%s: num_pages (%d) must be > 0", fn, num_pages);
  if ((int64_t)num_pages * page_size >= ((int64_t)1 << 31))
    return fail(TL_ERR_UNSUPPORTED, "%s: num_pages * page_size must be < 2^31", fn);
  if ((int64_t)batch * tokens_per_row >= ((int64_t)1 << 31))
    return fail(TL_ERR_UNSUPPORTED, "%s: batch * tokens_per_row must be < 2^31", fn);
  if (batch == 0 || tokens_per_row == 0) return ok();
  if (!tables) return fail(TL_ERR_INVALID, "%s: tables is NULL", fn);
  if (!positions) return fail(TL_ERR_INVALID, "%s: positions is NULL", fn);
  if (!slots) return fail(TL_ERR_INVALID, "%s: slots is NULL", fn);
  if (!aligned(tables, 4) || !aligned(positions, 4) || !aligned(slots, 4))
    return fail(TL_ERR_INVALID, "%s: tables/positions/slots are not 4-byte aligned", fn);
  hipStream_t s = (hipStream_t)stream;
  int rc;
  if (validate_mode()) {
    std::vector<int32_t> pos, tab;
    if ((rc = copy_to_host(fn, "positions", positions, (size_t)batch * tokens_per_row, pos, s))) return rc;
    if ((rc = copy_to_host(fn, "tables", tables, (size_t)batch * width, tab, s))) return rc;
    for (int32_t b = 0; b < batch; ++b)
      for (int32_t t = 0; t < tokens_per_row; ++t) {
        const int32_t p = pos[(size_t)b * tokens_per_row + t];
        if (p < 0) continue;
        int64_t blk = p / page_size;
        if (ring_pages > 0) blk %= ring_pages;
        if (blk >= width)
          return fail(TL_ERR_INVALID, "%s: positions[%d][%d] = %d is past the table (TL_VALIDATE)", fn, b, t, p);
        const int32_t page = tab[(size_t)b * width + blk];
        if (page < 0 || page >= num_pages)
          return fail(TL_ERR_INVALID, "%s: tables[%d][%lld] = %d is not a page of the pool (TL_VALIDATE)", fn, b,
                      (long long)blk, page);
      }
  }
  tl::SlotMapArgs a;
  a.tables = tables; a.positions = positions; a.slots = slots;
  a.batch = batch; a.tokens = tokens_per_row; a.width = width; a.ring = ring_pages;
  a.page_shift = log2i(page_size); a.num_pages = num_pages;
  hipError_t e = tl::launch_slot_mapping(a, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int tl_kv_gather(const tl_kv_pool* pool, const int32_t* block_table_row, int32_t length, void* k_out, void* v_out,
                 float* k_scale_out, float* v_scale_out, void* stream) {
  const char* fn = "tl_kv_gather";
  int rc = check_pool(fn, pool);
  if (rc) return rc;
  if (length < 0) return fail(TL_ERR_INVALID, "%s: length (%d) must be >= 0", fn, length);
  if (length == 0) return ok();
  if (!block_table_row) return fail(TL_ERR_INVALID, "%s: block_table_row is NULL", fn);
  if (!k_out) return fail(TL_ERR_INVALID, "%s: k_out is NULL", fn);
  if (!v_out) return fail(TL_ERR_INVALID, "%s: v_out is NULL", fn);
  if (!aligned(k_out, 16) || !aligned(v_out, 16)) return fail(TL_ERR_INVALID, "%s: k_out/v_out not 16-byte aligned", fn);
  if ((pool->dtype == TL_KV_FP8_E4M3 || pool->dtype == TL_KV_INT8) && (!k_scale_out || !v_scale_out))
    return fail(TL_ERR_INVALID, "%s: k_scale_out/v_scale_out are NULL for a scaled fp8 pool", fn);
  hipStream_t s = (hipStream_t)stream;
  tl::GatherArgs a;
  a.pool = pool_args(pool);
  a.table = block_table_row; a.length = length;
  a.k_out = k_out; a.v_out = v_out; a.k_scale_out = k_scale_out; a.v_scale_out = v_scale_out;
  hipError_t e = tl::launch_gather(a, pool->dtype, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

}  // extern "C"
