// readsum.hip -- the streaming-read reference kernel, for gfx950.
//
// Sums the 32-bit words of one buffer, read the way the fingerprint scan reads
// the body of a work item of a list of large items (one workgroup per 1 MiB
// chunk, one workgroup per CU, non-pipelined rounds of non-temporal 16-byte
// loads), with one add per word in place of the fingerprint's arithmetic.
// Its rounds hold 8 loads per lane instead of the scan's 12: with nothing to
// compute between rounds, 8 is the fastest depth measured (7.41-7.42 TB/s
// over 32 GiB, against 7.31 with 12 and 7.28 with pipelined rounds).  Like
// the scan's split tensors, each workgroup writes a partial result and a
// second launch merges them (a single shared atomic per workgroup instead
// costs about 15 % of the rate: every workgroup's update of one address is
// serialised across the XCDs).  Its rate is the streaming-read bandwidth the
// chip reaches with that load structure over one buffer of random words: a
// reference the scans' bandwidth is read against, not an upper bound (the
// list scan over a model's parameters has measured up to 1.2 % above it in
// the same run).
#include "scan_device.h"

namespace sdc {
namespace {

constexpr uint32_t kReadChunk = 1u << 20;
constexpr uint32_t kReadChunkVecs = kReadChunk / kVecBytes;
constexpr int kReadU = 8;
constexpr int kMergeThreads = 1024;

uint64_t read_chunks(uint64_t bytes) {
  const uint64_t nvec = bytes / kVecBytes;
  return nvec ? (nvec + kReadChunkVecs - 1) / kReadChunkVecs : 1u;
}

__global__ void __launch_bounds__(kBlock)
    read_sum_kernel(const unsigned char* buf, uint64_t nvec, uint32_t ntail, uint64_t* partial) {
  const uint32_t t = threadIdx.x;
  const uint64_t v0 = (uint64_t)blockIdx.x * kReadChunkVecs;
  const uint32_t nv = (uint32_t)min<uint64_t>(nvec - v0, kReadChunkVecs);
  uint64_t s = 0;
  if (nv) {
    stream_body<kReadU, false>(buf + v0 * kVecBytes, nv, [&](u32x4 v) {
      s += (uint64_t)v.x + (uint64_t)v.y + (uint64_t)v.z + (uint64_t)v.w;
    });
  }
  if (blockIdx.x == 0 && t < ntail)  // the last 0..3 words, past the last whole vector
    s += load_elem<4>(buf + nvec * kVecBytes + t * 4u);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __shared__ uint64_t ls[kWaves];
  if ((t & 63) == 0) ls[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < kWaves; ++i) s += ls[i];
    partial[blockIdx.x] = s;
  }
}

// One workgroup: *sum = the n partial sums, kMergeUnroll loads per lane in flight.
__global__ void __launch_bounds__(kMergeThreads)
    read_merge_kernel(const uint64_t* __restrict__ partial, uint32_t n, uint64_t* sum) {
  const uint32_t t = threadIdx.x;
  uint64_t s = 0;
  for (uint32_t i0 = 0; i0 < n; i0 += kMergeThreads * kMergeUnroll) {
    uint64_t v[kMergeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) {
      const uint32_t i = i0 + u * kMergeThreads + t;
      v[u] = (i < n) ? partial[i] : 0u;
    }
#pragma unroll
    for (uint32_t u = 0; u < kMergeUnroll; ++u) s += v[u];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __shared__ uint64_t ls[kMergeThreads / 64];
  if ((t & 63) == 0) ls[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < kMergeThreads / 64; ++i) s += ls[i];
    *sum = s;
  }
}

}  // namespace
}  // namespace sdc

using namespace sdc;

extern "C" int32_t sdc_read_sum_ws_bytes(uint64_t bytes, uint64_t* h_ws_bytes) {
  if (!h_ws_bytes) return SDC_ERR_INVALID;
  const uint64_t chunks = read_chunks(bytes);
  if (chunks > 0x7FFFFFFFull) return SDC_ERR_RANGE;
  *h_ws_bytes = chunks * sizeof(uint64_t);
  return SDC_OK;
}

extern "C" int32_t sdc_read_sum(const void* d_buf, uint64_t bytes, void* d_ws, uint64_t ws_bytes,
                                uint64_t* d_sum, sdc_stream_t stream) {
  if (!d_sum || !d_ws || (bytes && !d_buf) || bytes % 4u) return SDC_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(d_buf) % kVecBytes || reinterpret_cast<uintptr_t>(d_ws) % 8u)
    return SDC_ERR_ALIGN;
  uint64_t need = 0;
  int32_t st = sdc_read_sum_ws_bytes(bytes, &need);
  if (st) return st;
  if (ws_bytes < need) return SDC_ERR_WORKSPACE;
  const uint64_t chunks = read_chunks(bytes);
  hipStream_t s = as_stream(stream);
  uint64_t* partial = static_cast<uint64_t*>(d_ws);
  hipLaunchKernelGGL(read_sum_kernel, dim3((uint32_t)chunks), dim3(kBlock), kWideLdsBytes, s,
                     static_cast<const unsigned char*>(d_buf), bytes / kVecBytes,
                     (uint32_t)((bytes % kVecBytes) / 4u), partial);
  if ((st = launch_status())) return st;
  hipLaunchKernelGGL(read_merge_kernel, dim3(1), dim3(kMergeThreads), 0, s, partial,
                     (uint32_t)chunks, d_sum);
  return launch_status();
}
