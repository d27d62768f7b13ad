// Host page allocator for the page pool, and the device page copy its copy-on-write
// needs.  The allocator follows the backend rules of "How serving works in Tlaloc"
// (the runtime comparison table and the section 3 backend bullets): pages are held
// per sequence and freed when it ends; when pages run short they are reclaimed only
// from sequences idle past the timeout, least recently active first and only as many
// as needed; otherwise the request is refused by name, listing the holders, and the
// refused sequence keeps its pages (the refusal counts as activity).  Prefix sharing
// (the KV-cache management page, "Reuse identical causal prefixes" and the paragraph
// before it): a forked sequence shares its parent's prefix pages with reference
// counts, and a shared, partly filled last page is copied before either holder writes
// into it.  The lowest free page is always taken first, so the decisions are
// deterministic.  Not thread-safe: one allocator per host thread (or a caller lock).
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <map>
#include <set>
#include <string>
#include <vector>

#include "tl_internal.h"

struct tl_page_allocator {
  struct Seq {
    int64_t len = 0;
    std::vector<int32_t> pages;
    double last = 0.0;
  };
  int32_t page_size = 0;
  double timeout = 0.0;
  std::vector<int32_t> ref;       // holders of each page
  std::set<int32_t> free_pages;   // pages with no holder, lowest first
  std::map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t p = *free_pages.begin();
    free_pages.erase(free_pages.begin());
    ref[p] = 1;
    return p;
  }
  void drop(int32_t p) {
    if (--ref[p] == 0) free_pages.insert(p);
  }
  void release(int64_t id) {
    for (int32_t p : seqs[id].pages) drop(p);
    seqs.erase(id);
  }
};

namespace {

int afail(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return tl::set_error(code, buf);
}

// K, V and (scaled pools) scales of page src[i] -> page dst[i]; 16 bytes a thread
__global__ __launch_bounds__(256) void copy_pages_kernel(tl::CopyPagesArgs p, const int32_t* src, const int32_t* dst) {
  const int i = blockIdx.y;
  const int s = src[i], d = dst[i];
  if (s < 0 || s >= p.num_pages || d < 0 || d >= p.num_pages) return;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u < p.units) {
    reinterpret_cast<uint4*>(p.k)[d * p.units + u] = reinterpret_cast<const uint4*>(p.k)[s * p.units + u];
    reinterpret_cast<uint4*>(p.v)[d * p.units + u] = reinterpret_cast<const uint4*>(p.v)[s * p.units + u];
  }
  if (p.k_scale && u < p.scales) {
    p.k_scale[d * p.scales + u] = p.k_scale[s * p.scales + u];
    p.v_scale[d * p.scales + u] = p.v_scale[s * p.scales + u];
  }
}

}  // namespace

namespace tl {
hipError_t launch_copy_pages(const CopyPagesArgs& p, const int32_t* src, const int32_t* dst, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t per = std::max(p.units, p.scales);
  hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)((per + 255) / 256), (unsigned)n), dim3(256), 0, s, p, src, dst);
  return hipGetLastError();
}
}  // namespace tl

extern "C" {

tl_page_allocator* tl_alloc_create(int32_t num_pages, int32_t page_size, double idle_timeout) {
  if (num_pages <= 0 || page_size <= 0) {
    afail(TL_ERR_INVALID, "tl_alloc_create: num_pages (%d) and page_size (%d) must be > 0", num_pages, page_size);
    return nullptr;
  }
  tl_page_allocator* a = new tl_page_allocator();
  a->page_size = page_size;
  a->timeout = idle_timeout;
  a->ref.assign(num_pages, 0);
  for (int32_t p = 0; p < num_pages; ++p) a->free_pages.insert(a->free_pages.end(), p);
  tl::set_error(TL_OK, "");
  return a;
}

void tl_alloc_destroy(tl_page_allocator* a) { delete a; }

int32_t tl_alloc_free_pages(const tl_page_allocator* a) { return a ? (int32_t)a->free_pages.size() : -1; }

int tl_alloc_start(tl_page_allocator* a, int64_t seq, double now) {
  if (!a) return afail(TL_ERR_INVALID, "tl_alloc_start: allocator is NULL");
  if (a->seqs.count(seq)) return afail(TL_ERR_INVALID, "tl_alloc_start: sequence %lld is already started", (long long)seq);
  a->seqs[seq].last = now;
  return tl::set_error(TL_OK, "");
}

int tl_alloc_end(tl_page_allocator* a, int64_t seq) {
  if (!a) return afail(TL_ERR_INVALID, "tl_alloc_end: allocator is NULL");
  if (!a->seqs.count(seq)) return afail(TL_ERR_INVALID, "tl_alloc_end: sequence %lld is not started", (long long)seq);
  a->release(seq);
  return tl::set_error(TL_OK, "");
}

int tl_alloc_fork(tl_page_allocator* a, int64_t parent, int64_t child, int64_t n_tokens, double now) {
  const char* fn = "tl_alloc_fork";
  if (!a) return afail(TL_ERR_INVALID, "%s: allocator is NULL", fn);
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return afail(TL_ERR_INVALID, "%s: sequence %lld is not started", fn, (long long)parent);
  if (a->seqs.count(child)) return afail(TL_ERR_INVALID, "%s: sequence %lld is already started", fn, (long long)child);
  if (n_tokens < 0 || n_tokens > it->second.len)
    return afail(TL_ERR_INVALID, "%s: prefix of %lld tokens is outside sequence %lld", fn, (long long)n_tokens,
                 (long long)parent);
  const size_t np = (size_t)((n_tokens + a->page_size - 1) / a->page_size);
  std::vector<int32_t> pages(it->second.pages.begin(), it->second.pages.begin() + np);
  for (int32_t p : pages) ++a->ref[p];
  it->second.last = now;
  tl_page_allocator::Seq& c = a->seqs[child];
  c.len = n_tokens;
  c.pages = pages;
  c.last = now;
  return tl::set_error(TL_OK, "");
}

int tl_alloc_append(tl_page_allocator* a, int64_t seq, int32_t n_tokens, double now, int32_t* slots_out,
                    int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies) {
  const char* fn = "tl_alloc_append";
  if (!a) return afail(TL_ERR_INVALID, "%s: allocator is NULL", fn);
  if (n_tokens < 0) return afail(TL_ERR_INVALID, "%s: n_tokens (%d) must be >= 0", fn, n_tokens);
  if ((n_tokens > 0 && !slots_out) || !copy_src || !copy_dst || !n_copies)
    return afail(TL_ERR_INVALID, "%s: an output array is NULL", fn);
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return afail(TL_ERR_INVALID, "%s: sequence %lld is not started", fn, (long long)seq);
  tl_page_allocator::Seq& s = it->second;
  const int64_t S = a->page_size, L = s.len;
  const int64_t new_pages = (L + n_tokens + S - 1) / S - (int64_t)s.pages.size();
  const bool cow = n_tokens > 0 && L % S != 0 && a->ref[s.pages.back()] > 1;
  const int64_t need = new_pages + (cow ? 1 : 0);
  const int64_t free = (int64_t)a->free_pages.size();
  if (need > free) {
    // idle sequences, least recently active first; reclaim only if they cover the shortage
    std::vector<std::pair<double, int64_t>> idle;
    for (auto& kv : a->seqs)
      if (kv.first != seq && kv.second.last < now - a->timeout) idle.push_back({kv.second.last, kv.first});
    std::sort(idle.begin(), idle.end());
    std::vector<int32_t> ref = a->ref;
    int64_t gain = 0;
    std::vector<int64_t> take;
    for (auto& c : idle) {
      if (free + gain >= need) break;
      for (int32_t p : a->seqs[c.second].pages) gain += (--ref[p] == 0);
      take.push_back(c.second);
    }
    if (free + gain < need) {
      s.last = now;  // a refused request still counts as activity
      std::string held;
      for (auto& kv : a->seqs) {
        if (kv.second.pages.empty()) continue;
        if (!held.empty()) held += ", ";
        held += std::to_string(kv.first) + " (" + std::to_string(kv.second.pages.size()) + " pages)";
      }
      return afail(TL_ERR_NO_PAGES, "%s: sequence %lld needs %lld pages, %lld free; held by: %s", fn, (long long)seq,
                   (long long)need, (long long)free, held.c_str());
    }
    for (int64_t i : take) a->release(i);
  }
  tl_page_allocator::Seq& t = a->seqs[seq];  // (the map may have changed)
  *n_copies = 0;
  if (cow) {
    const int32_t old = t.pages.back();
    const int32_t nw = a->take();
    a->drop(old);
    t.pages.back() = nw;
    copy_src[0] = old;
    copy_dst[0] = nw;
    *n_copies = 1;
  }
  for (int64_t i = 0; i < new_pages; ++i) t.pages.push_back(a->take());
  for (int64_t p = L; p < L + n_tokens; ++p) slots_out[p - L] = (int32_t)(t.pages[p / S] * S + p % S);
  t.len = L + n_tokens;
  t.last = now;
  return tl::set_error(TL_OK, "");
}

int tl_alloc_tables(const tl_page_allocator* a, const int64_t* seqs, int32_t n, int32_t max_blocks, int32_t* tables,
                    int32_t* lens) {
  const char* fn = "tl_alloc_tables";
  if (!a) return afail(TL_ERR_INVALID, "%s: allocator is NULL", fn);
  if (n < 0 || max_blocks <= 0) return afail(TL_ERR_INVALID, "%s: n (%d) or max_blocks (%d) out of range", fn, n, max_blocks);
  if (n > 0 && (!seqs || !tables || !lens)) return afail(TL_ERR_INVALID, "%s: an array is NULL", fn);
  for (int32_t b = 0; b < n; ++b) {
    auto it = a->seqs.find(seqs[b]);
    if (it == a->seqs.end()) return afail(TL_ERR_INVALID, "%s: sequence %lld is not started", fn, (long long)seqs[b]);
    const auto& p = it->second.pages;
    if ((int64_t)p.size() > max_blocks)
      return afail(TL_ERR_INVALID, "%s: sequence %lld holds %zu pages, more than %d", fn, (long long)seqs[b], p.size(),
                   max_blocks);
    for (int32_t j = 0; j < max_blocks; ++j) tables[(int64_t)b * max_blocks + j] = j < (int32_t)p.size() ? p[j] : -1;
    lens[b] = (int32_t)std::min<int64_t>(it->second.len, INT32_MAX);
  }
  return tl::set_error(TL_OK, "");
}

}  // extern "C"
