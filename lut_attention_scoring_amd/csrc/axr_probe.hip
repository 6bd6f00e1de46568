// Bandwidth probes: plain streaming kernels that move a given number of bytes
// with no arithmetic beyond a checksum.  They give the achievable HBM rate on
// the machine the kernels run on, so the method's kernels can be reported
// against both the published peak and what a bare stream reaches.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "axr_probe.h"

namespace {

constexpr int kThreads = 512;
constexpr int kReadBlocks = 4096;

// Grid-stride 16-byte loads; the xor checksum is written only if it hits an
// impossible value, so the loads cannot be dropped and nothing is stored.
__global__ __launch_bounds__(kThreads) void read_stream(const uint4* __restrict__ p, int64_t n16,
                                                       uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Each block reads a contiguous share of the input and then writes a
// contiguous share of the output (the shape of a scan that emits results).
__global__ __launch_bounds__(kThreads) void read_write_stream(const uint4* __restrict__ in,
                                                             int64_t n16_in,
                                                             uint32_t* __restrict__ out,
                                                             int64_t n4_out) {
  const int64_t per_in = (n16_in + gridDim.x - 1) / gridDim.x;
  const int64_t per_out = (n4_out + gridDim.x - 1) / gridDim.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * per_in;
  const int64_t i1 = i0 + per_in < n16_in ? i0 + per_in : n16_in;
  const int64_t o0 = static_cast<int64_t>(blockIdx.x) * per_out;
  const int64_t o1 = o0 + per_out < n4_out ? o0 + per_out : n4_out;
  uint32_t acc = 0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += kThreads) {
    const uint4 v = in[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int64_t o = o0 + threadIdx.x; o < o1; o += kThreads) out[o] = acc + static_cast<uint32_t>(o);
}

// LDS table-read loop: every thread owns 16 addresses in the score kernel's
// pattern (row from a per-lane xorshift hash, column (step + key slot + 4u)
// mod 16 for lane u of a 4-lane key); each pass xors a uniform value into the
// row bits, which keeps the columns and moves the rows.  Every address is
// masked to the 128 KiB array.
constexpr int kLdsEntries = 8192;   // 16-byte entries
__global__ __launch_bounds__(1024) void lds_read(int iters, uint32_t* __restrict__ out) {
  __shared__ uint4 tab[kLdsEntries];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsEntries; i += 1024)
    tab[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
  __syncthreads();
  const uint32_t lane = tid % 64, u = lane % 4, kslot = (lane / 4) % 4;
  uint32_t h = 0x9E3779B9u ^ (static_cast<uint32_t>(tid + 1024 * blockIdx.x) * 0x85EBCA6Bu);
  uint32_t addr[16];
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    addr[st] = u * 32768u + ((h >> 9) & 127u) * 256u + 16u * ((st + kslot + 4u * u) & 15u);
  }
  uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  const char* base = reinterpret_cast<const char*>(tab);
  for (int it = 0; it < iters; ++it) {
    const uint32_t r = ((static_cast<uint32_t>(it) * 0x35u) & 127u) << 8;
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const uint4 e = *reinterpret_cast<const uint4*>(base + ((addr[st] ^ r) & (kLdsEntries * 16u - 16u)));
      a0 += e.x;
      a1 += e.y;
      a2 += e.z;
      a3 += e.w;
    }
  }
  out[blockIdx.x * 1024 + tid] = a0 ^ a1 ^ a2 ^ a3;
}

}  // namespace

extern "C" int axr_probe_lds_read(int iters, uint32_t* out, void* stream) {
  if (out == nullptr || iters < 1 || iters > 65536 || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return -1;
  hipLaunchKernelGGL(lds_read, dim3(256), dim3(1024), 0, static_cast<hipStream_t>(stream), iters,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int axr_probe_read_stream(const void* buf, int64_t bytes, uint32_t* sink,
                                     void* stream) {
  if (buf == nullptr || sink == nullptr || bytes < 0 || (bytes & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return -1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(read_stream, dim3(kReadBlocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int axr_probe_read_write(const void* in, int64_t in_bytes, void* out,
                                    int64_t out_bytes, void* stream) {
  if (in == nullptr || out == nullptr || in_bytes < 0 || out_bytes < 0 || (in_bytes & 15) != 0 ||
      (out_bytes & 3) != 0 || (reinterpret_cast<uintptr_t>(in) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return -1;
  if (in_bytes == 0 && out_bytes == 0) return 0;
  // ~16 KiB moved per block: the fastest grid measured for both a 143 MB and
  // a 646 MB stream (fewer, longer blocks finish unevenly; more spend their
  // time starting up)
  int64_t blocks = (in_bytes + out_bytes) / (16 * 1024);
  blocks = blocks < 256 ? 256 : (blocks > 65535 ? 65535 : blocks);
  hipLaunchKernelGGL(read_write_stream, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(in),
                     in_bytes / 16, static_cast<uint32_t*>(out), out_bytes / 4);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
