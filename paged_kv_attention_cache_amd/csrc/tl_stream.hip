// Streaming-read ceiling of HBM on this GPU: every 16-byte unit of a buffer is read
// once, with plain or nontemporal loads (the decode kernels read the KV pages with
// nontemporal loads).  This is measurement support for the roofline figures, built as
// its own small library (libtl_stream.so) beside libtl.so; the attention path never
// calls it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u4 ld(const u4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p); else return *p;
}

// Each thread reads four units per trip, a grid stride apart, and folds them into one
// word; the word is stored only if it equals a value the data never produces here, so
// the loads stay live without any real store traffic.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u4* p, int64_t units, unsigned* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < units; i += 4 * stride) {
    const u4 a = ld<NT>(p + i), b = ld<NT>(p + i + stride), c = ld<NT>(p + i + 2 * stride),
             d = ld<NT>(p + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < units; i += stride) {
    const u4 a = ld<NT>(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Blocks of 4 KiB (256 units) read in the order a list gives, as a paged decode reads
// a (page, head) span of K or V: each workgroup takes four blocks per trip (one unit
// per thread of each), so four loads per thread are in flight.
template <bool NT>
__global__ __launch_bounds__(256) void block_read_kernel(const u4* p, const int32_t* blocks, int64_t n_blocks,
                                                         unsigned* sink) {
  unsigned acc = 0;
  int64_t b = (int64_t)blockIdx.x * 4;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (; b + 3 < n_blocks; b += stride) {
    const u4 x0 = ld<NT>(p + (int64_t)blocks[b] * 256 + threadIdx.x);
    const u4 x1 = ld<NT>(p + (int64_t)blocks[b + 1] * 256 + threadIdx.x);
    const u4 x2 = ld<NT>(p + (int64_t)blocks[b + 2] * 256 + threadIdx.x);
    const u4 x3 = ld<NT>(p + (int64_t)blocks[b + 3] * 256 + threadIdx.x);
    acc ^= x0[0] ^ x0[1] ^ x0[2] ^ x0[3] ^ x1[0] ^ x1[1] ^ x1[2] ^ x1[3] ^ x2[0] ^ x2[1] ^ x2[2] ^ x2[3] ^ x3[0] ^
           x3[1] ^ x3[2] ^ x3[3];
  }
  for (; b < n_blocks; ++b) {
    const u4 x0 = ld<NT>(p + (int64_t)blocks[b] * 256 + threadIdx.x);
    acc ^= x0[0] ^ x0[1] ^ x0[2] ^ x0[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// The same shuffled blocks with U loads per thread in flight at once: each trip
// issues U loads (U blocks, one unit per thread of each) before it uses any, so a
// wave keeps U KiB in flight.  Launched as a persistent grid whose workgroups per CU
// the caller caps with dynamic LDS, it shows how many bytes in flight per CU the
// memory system needs to run at full rate.
template <int U>
__global__ __launch_bounds__(256) void block_depth_kernel(const u4* p, const int32_t* blocks, int64_t n_blocks,
                                                          unsigned* sink) {
  unsigned acc = 0;
  for (int64_t b = (int64_t)blockIdx.x * U; b + U - 1 < n_blocks; b += (int64_t)gridDim.x * U) {
    u4 x[U];
#pragma unroll
    for (int j = 0; j < U; ++j) x[j] = __builtin_nontemporal_load(p + (int64_t)blocks[b + j] * 256 + threadIdx.x);
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= x[j][0] ^ x[j][1] ^ x[j][2] ^ x[j][3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Mixed reads and writes: each thread reads R units (a stride of out_units apart) and
// writes one, their XOR, per trip.  R = 1 is a copy; R = 2 and 4 read as many bytes per
// byte written as a KV write into bf16 and into 1-byte pools does.
template <int R, bool NTL, bool NTS>
__global__ __launch_bounds__(256) void stream_rw_kernel(const u4* src, u4* dst, int64_t out_units) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < out_units; i += stride) {
    u4 x = ld<NTL>(src + i);
#pragma unroll
    for (int r = 1; r < R; ++r) x ^= ld<NTL>(src + i + r * out_units);
    if constexpr (NTS) __builtin_nontemporal_store(x, dst + i); else dst[i] = x;
  }
}

template <int R>
int launch_rw(const u4* src, u4* dst, int64_t out_units, int ntl, int nts, int wgs, hipStream_t s) {
  if (ntl && !nts) hipLaunchKernelGGL((stream_rw_kernel<R, true, false>), dim3(wgs), dim3(256), 0, s, src, dst, out_units);
  else if (!ntl && nts) hipLaunchKernelGGL((stream_rw_kernel<R, false, true>), dim3(wgs), dim3(256), 0, s, src, dst, out_units);
  else if (ntl && nts) hipLaunchKernelGGL((stream_rw_kernel<R, true, true>), dim3(wgs), dim3(256), 0, s, src, dst, out_units);
  else hipLaunchKernelGGL((stream_rw_kernel<R, false, false>), dim3(wgs), dim3(256), 0, s, src, dst, out_units);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// Read ratio * out_bytes at src and write out_bytes at dst (ratio 1, 2 or 4; both
// 16-byte aligned, out_bytes a multiple of 16, the two ranges disjoint), with plain
// or nontemporal loads and stores.  Returns 0, -1 for an unsupported ratio, or the
// launch's HIP error.
int tl_stream_rw(const void* src, void* dst, size_t out_bytes, int ratio, int nt_loads, int nt_stores, int workgroups,
                 void* stream) {
  const int64_t units = (int64_t)(out_bytes / 16);
  if (units <= 0 || workgroups <= 0) return 0;
  const u4* p = static_cast<const u4*>(src);
  u4* q = static_cast<u4*>(dst);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (ratio) {
    case 1: return launch_rw<1>(p, q, units, nt_loads, nt_stores, workgroups, s);
    case 2: return launch_rw<2>(p, q, units, nt_loads, nt_stores, workgroups, s);
    case 4: return launch_rw<4>(p, q, units, nt_loads, nt_stores, workgroups, s);
    default: return -1;
  }
}

// Read the blocks blocks[0 .. n_blocks - 1] (4 KiB each, as in tl_block_read) with
// `depth` (4, 8, 16 or 32) loads per thread in flight, on `workgroups` workgroups of
// 256 threads with lds_bytes of dynamic LDS each (to cap the workgroups per CU).
// Blocks past the last whole trip of the grid are not read.  Returns 0, -1 for an
// unsupported depth, or the launch's HIP error.
int tl_block_read_depth(const void* src, const int32_t* blocks, int64_t n_blocks, unsigned* sink, int depth,
                        int workgroups, int lds_bytes, void* stream) {
  if (n_blocks <= 0 || workgroups <= 0) return 0;
  const u4* p = static_cast<const u4*>(src);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (depth) {
    case 4: hipLaunchKernelGGL(block_depth_kernel<4>, dim3((unsigned)workgroups), dim3(256), lds_bytes, s, p, blocks, n_blocks, sink); break;
    case 8: hipLaunchKernelGGL(block_depth_kernel<8>, dim3((unsigned)workgroups), dim3(256), lds_bytes, s, p, blocks, n_blocks, sink); break;
    case 16: hipLaunchKernelGGL(block_depth_kernel<16>, dim3((unsigned)workgroups), dim3(256), lds_bytes, s, p, blocks, n_blocks, sink); break;
    case 32: hipLaunchKernelGGL(block_depth_kernel<32>, dim3((unsigned)workgroups), dim3(256), lds_bytes, s, p, blocks, n_blocks, sink); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

// Read n_blocks blocks of 4 KiB of `src` in the order blocks[] (device int32 block
// indices, each < bytes of src / 4096) gives.  Returns 0 or the launch's HIP error.
int tl_block_read(const void* src, const int32_t* blocks, int64_t n_blocks, unsigned* sink, int nontemporal,
                  int workgroups, void* stream) {
  if (n_blocks <= 0 || workgroups <= 0) return 0;
  const u4* p = static_cast<const u4*>(src);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(block_read_kernel<true>, dim3((unsigned)workgroups), dim3(256), 0, s, p, blocks, n_blocks, sink);
  else
    hipLaunchKernelGGL(block_read_kernel<false>, dim3((unsigned)workgroups), dim3(256), 0, s, p, blocks, n_blocks, sink);
  return (int)hipGetLastError();
}

// Read `bytes` (a multiple of 16, 16-byte aligned) of device memory at `src` once.
// sink: one device word, written only in the unlikely case above.  Returns 0, or the
// HIP error code of the launch.
int tl_stream_read(const void* src, size_t bytes, unsigned* sink, int nontemporal, int workgroups, void* stream) {
  const int64_t units = (int64_t)(bytes / 16);
  if (units <= 0 || workgroups <= 0) return 0;
  const u4* p = static_cast<const u4*>(src);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)workgroups), dim3(256), 0, s, p, units, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)workgroups), dim3(256), 0, s, p, units, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
