// Achievable-peak probes for gfx950 (measurement only, not the DSA path):
// matrix-core issue loops and a streaming HBM read.  See include/dsa_probe.h.
#include "common.h"
#include "dsa_probe.h"

namespace dsa {

constexpr int kChains = 8;  // independent accumulators per wave (hide the MFMA latency)

template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  float r = 0.f;
  if constexpr (KIND == 0) {
    // small e4m3 codes (0x30 | lane bits): finite, no saturation over the loop
    const int pat = 0x30303030 | (lane & 7);
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = pat + i;
      b[i] = pat ^ (i << 8);
    }
    v4f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma_fp8_16x16x128(a, b, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][0] + acc[c][3];
  } else if constexpr (KIND == 1) {
    v8s a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (short)(0x3F80 + (lane & 7));
      b[i] = (short)(0x3C00 + i);
    }
    v4f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = (v4f){0.f, 0.f, 0.f, 0.f};
    // two MFMAs per chain per iteration (the accumulators then keep their
    // registers across the loop; with one, the compiler rotated them through
    // register copies that wait on every result)
    for (int64_t it = 0; it < iters; it += 2) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[c] = mfma_bf16_16x16x32(a, b, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][0] + acc[c][3];
  } else {
    v8s a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (short)(0x3F80 + (lane & 7));
      b[i] = (short)(0x3C00 + i);
    }
    v16f acc[kChains / 2];
#pragma unroll
    for (int c = 0; c < kChains / 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains / 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((v8bf)a, (v8bf)b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChains / 2; ++c) r += acc[c][0] + acc[c][15];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = r;
}

// Streaming read: block b reads its own contiguous 1/gridDim of the buffer,
// eight 16-byte non-temporal loads in flight per thread (the fastest of the
// read patterns measured: 7.0-7.2 TB/s, against 6.2 TB/s with ordinary loads
// and 5.3-5.6 TB/s for a grid-strided loop).
__global__ __launch_bounds__(256) void probe_read_kernel(const v4i* __restrict__ buf, int64_t per_block,
                                                         float* __restrict__ sink) {
  constexpr int U = 8;
  const v4i* p = buf + (int64_t)blockIdx.x * per_block + threadIdx.x;
  int x = 0;
  for (int64_t i = 0; i < per_block; i += 256 * U) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + 256 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = (float)(x & 0xFFFF);
}

}  // namespace dsa

using namespace dsa;

extern "C" {

static const double kMfmaFlops[3] = {65536.0, 16384.0, 32768.0};

double dsa_probe_mfma_flops(int kind, int64_t iters, int64_t blocks) {
  if (kind < 0 || kind > 2 || iters < 0 || blocks < 1) return 0.0;
  // 4 waves per block, 8 instructions per wave and round
  return kMfmaFlops[kind] * 8.0 * 4.0 * (double)iters * (double)blocks;
}

int dsa_probe_mfma(int kind, int64_t iters, int64_t blocks, float* sink, void* stream) {
  if (kind < 0 || kind > 2 || iters < 0 || (iters & 1) || blocks < 1 || blocks > 2147483647 || !sink) return -1;
  hipStream_t st = (hipStream_t)stream;
  if (kind == 0) probe_mfma_kernel<0><<<(unsigned)blocks, 256, 0, st>>>(iters, sink);
  else if (kind == 1) probe_mfma_kernel<1><<<(unsigned)blocks, 256, 0, st>>>(iters, sink);
  else probe_mfma_kernel<2><<<(unsigned)blocks, 256, 0, st>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int dsa_probe_read(const void* buf, int64_t bytes, int64_t blocks, float* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || blocks < 1 || blocks > 2147483647 || bytes % 16) return -1;
  if ((bytes / 16) % (blocks * 256 * 8)) return -1;
  probe_read_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>((const v4i*)buf, bytes / 16 / blocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
