// Streaming probe: what HBM delivers on this machine for the compressor's
// traffic (two raw bf16 arrays of T rows x 512 read once; one 1 KB entry row
// written per 4 rows and one per 128 rows), with none of its arithmetic.
// A measurement tool, not part of the attention path: it bounds what any
// kernel with this read/write mix can reach.
//
// Layout of the work as in the fused compressor: 256 blocks of 16 waves,
// each wave streaming a contiguous range of rows, one 16-byte load a lane
// per row and array, eight rows in flight.  The rows are read with
// non-temporal loads, as the compressor reads them (read once, no cache
// allocation); the entry rows are written with ordinary stores.  Modes:
//   0  reads only
//   1  reads, with the entry rows written as the rows stream (the mix)
//   2  the entry-row writes only
//   3  reads, then each wave's entry rows written after all of its reads
// The loaded words are folded into a checksum (written per wave, so the
// loads are not removed); written rows carry the running checksum.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWaves = 16, kDepth = 8;

__global__ __launch_bounds__(64 * kWaves) void stream_probe_kernel(const uint4* __restrict__ x,
                                                                   const uint4* __restrict__ z,
                                                                   int64_t rows, uint4* __restrict__ o4,
                                                                   uint4* __restrict__ o128, int mode,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t per = (rows + nw - 1) / nw;                   // a multiple of 128 for the probed sizes
  const int64_t r0 = wave * per, r1 = r0 + per < rows ? r0 + per : rows;
  uint32_t acc = 0;
  auto fold = [&](uint4 v) { acc ^= v.x ^ (v.y << 1) ^ (v.z << 2) ^ (v.w << 3); };
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  auto ld = [](const uint4* p) {
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
  };
  auto put = [&](int64_t r) {                                 // entry rows closed at row r
    const uint4 w = make_uint4(acc, acc + 1, acc + 2, acc + 3);
    if ((r & 3) == 3) o4[(r >> 2) * 64 + lane] = w;
    if ((r & 127) == 127) o128[(r >> 7) * 64 + lane] = w;
  };
  if (mode == 2) {
    for (int64_t r = r0; r < r1; ++r) put(r);
  } else {
    uint4 bx[kDepth], bz[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int64_t r = r0 + i;
      if (r < r1) {
        bx[i] = ld(x + r * 64 + lane);
        bz[i] = ld(z + r * 64 + lane);
      }
    }
    for (int64_t rb = r0; rb < r1; rb += kDepth) {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        const int64_t r = rb + i;
        if (r < r1) {
          fold(bx[i]);
          fold(bz[i]);
          if (mode == 1) put(r);
          const int64_t rn = r + kDepth;
          if (rn < r1) {
            bx[i] = ld(x + rn * 64 + lane);
            bz[i] = ld(z + rn * 64 + lane);
          }
        }
      }
    }
    if (mode == 3)
      for (int64_t r = r0; r < r1; ++r) put(r);
  }
  if (lane == 0) sink[wave] = acc;
}

}  // namespace

extern "C" {

// mode 0..3 as above; x, z: rows x 512 bf16 (16-byte aligned); o4: rows / 4
// rows of 1 KB; o128: rows / 128 rows of 1 KB; sink: 4096 words.  rows must
// be a multiple of 4096 * 128.  Returns the HIP status of the launch.
int cskv_probe_stream(int mode, const void* x, const void* z, int64_t rows, void* o4, void* o128,
                      uint32_t* sink, void* stream) {
  if (mode < 0 || mode > 3 || rows <= 0 || rows % (4096 * 128) != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_probe_kernel, dim3(256), dim3(64 * kWaves), 0, (hipStream_t)stream,
                     (const uint4*)x, (const uint4*)z, rows, (uint4*)o4, (uint4*)o128, mode, sink);
  return (int)hipGetLastError();
}

}
