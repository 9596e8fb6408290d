// HBM probes of known byte counts (include/hqq_probe.h): a streaming device copy and a
// streaming read of up to three buffers, 16-byte non-temporal accesses, four or eight loads in
// flight per thread.  They compute nothing of the method; the measurements use them as the
// practical rate of a memory-bound kernel on the same device (copy: read + write; read: the
// floor of a kernel that only has to stream given buffers once) and as the copy of known size
// that calibrates the HBM byte counters.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hqq_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

// Block b copies 16-byte elements [b U T, (b + 1) U T): U loads per thread in flight, then the
// stores; only the last block takes the guarded path.
template <int U>
__global__ void __launch_bounds__(kThreads) k_probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
  u32x4 v[U];
  if (base + (int64_t)(U - 1) * kThreads < n) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + base + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + base + u * kThreads);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * kThreads < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + base + u * kThreads),
                                                               dst + base + u * kThreads);
  }
}

struct ReadSet {
  const u32x4* p[3];
  int64_t n[3];   // 16-byte elements
  int64_t b1, b2; // first block of buffers 1 and 2
};

// The blocks of buffer i follow those of buffer i - 1.  The loaded words are folded into one
// value that is stored only if it equals a constant, so the loads cannot be dropped and
// (practically) nothing is written.
template <int U>
__global__ void __launch_bounds__(kThreads) k_probe_read(const ReadSet rs, unsigned* __restrict__ sink) {
  const int64_t b = blockIdx.x;
  const int which = b >= rs.b2 ? 2 : (b >= rs.b1 ? 1 : 0);
  const int64_t lb = b - (which == 2 ? rs.b2 : (which == 1 ? rs.b1 : 0));
  const u32x4* p = rs.p[which];
  const int64_t n = rs.n[which];
  const int64_t base = lb * kThreads * U + threadIdx.x;
  unsigned acc = 0;
  if (base + (int64_t)(U - 1) * kThreads < n) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + base + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * kThreads < n) {
        const u32x4 v = __builtin_nontemporal_load(p + base + u * kThreads);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x & 3] = acc;
}

int64_t blocks_for(int64_t n, int U) { return (n + (int64_t)kThreads * U - 1) / ((int64_t)kThreads * U); }

}  // namespace

extern "C" {

int hqq_probe_copy(const void* src, void* dst, size_t bytes, int unroll, void* stream) {
  if (!src || !dst || (bytes & 15) || bytes == 0 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return 1;
  if (unroll != 4 && unroll != 8) return 1;
  const int64_t n = (int64_t)(bytes / 16);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (unroll == 4)
    hipLaunchKernelGGL(k_probe_copy<4>, dim3((unsigned)blocks_for(n, 4)), dim3(kThreads), 0, st,
                       reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n);
  else
    hipLaunchKernelGGL(k_probe_copy<8>, dim3((unsigned)blocks_for(n, 8)), dim3(kThreads), 0, st,
                       reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int hqq_probe_read(const void* const* bufs, const size_t* bytes, int nbuf, void* sink, int unroll, void* stream) {
  if (!bufs || !bytes || nbuf < 1 || nbuf > 3 || !sink || ((uintptr_t)sink & 15)) return 1;
  if (unroll != 4 && unroll != 8) return 1;
  ReadSet rs;
  int64_t blocks[3] = {0, 0, 0};
  for (int i = 0; i < 3; ++i) {
    if (i < nbuf) {
      if (!bufs[i] || (bytes[i] & 15) || bytes[i] == 0 || ((uintptr_t)bufs[i] & 15)) return 1;
      rs.p[i] = reinterpret_cast<const u32x4*>(bufs[i]);
      rs.n[i] = (int64_t)(bytes[i] / 16);
      blocks[i] = blocks_for(rs.n[i], unroll);
    } else {
      rs.p[i] = rs.p[0];
      rs.n[i] = 0;
    }
  }
  rs.b1 = blocks[0];
  rs.b2 = blocks[0] + blocks[1];
  const int64_t total = blocks[0] + blocks[1] + blocks[2];
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (unroll == 4)
    hipLaunchKernelGGL(k_probe_read<4>, dim3((unsigned)total), dim3(kThreads), 0, st, rs,
                       reinterpret_cast<unsigned*>(sink));
  else
    hipLaunchKernelGGL(k_probe_read<8>, dim3((unsigned)total), dim3(kThreads), 0, st, rs,
                       reinterpret_cast<unsigned*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
