// Fold W_index into the index query and re-quantise it to e4m3.
//
// The indexer score is q_t . W_index . k_s (DeepSeek-V3.2 write-up, section
// 2.2).  Folding W into q once per query turns the per-pair work into one
// 128-wide FP8 dot product; the folded row is re-quantised with its own
// amax/448 scale so that the pair product stays FP8.
//
// Work: T x 128 x 128 MACs in fp64 (bit-reproducible codes), ~1/1024 of the
// indexer's pair work.  Long prefills with a bf16 W run a register-tiled
// kernel (64 rows per block, 8 x 4 fp64 accumulators per thread); the fp32-W
// configuration has one thread own one output column j with column j of W in
// registers while a block walks its query rows held in LDS as fp64; short
// batches split each column's sum over four waves instead.
#include "common.h"
#include "kernels.h"

namespace dsa {

// kFoldRows query rows per block (32, for long prefills; short batches use
// fold_split_kernel below)
template <bool kFp8In, bool kWBf16, int kFoldRows>
__global__ __launch_bounds__(128) void fold_kernel(const void* __restrict__ q_in,
                                                   const float* __restrict__ q_scale,
                                                   const void* __restrict__ w_in, int64_t T,
                                                   void* __restrict__ q_out,
                                                   float* __restrict__ s_out) {
  __shared__ double qrow[kFoldRows][kIdxDim];
  __shared__ double wmax[2][kFoldRows];
  const int j = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kFoldRows;
  const int nr = (int)min<int64_t>(kFoldRows, T - r0);

  float wcol[kIdxDim];
#pragma unroll
  for (int i = 0; i < kIdxDim; ++i) {
    if (kWBf16)
      wcol[i] = bf16_to_f32(((const uint16_t*)w_in)[i * kIdxDim + j]);
    else
      wcol[i] = ((const float*)w_in)[i * kIdxDim + j];
  }
  for (int r = nr; r < kFoldRows; ++r) qrow[r][j] = 0.0;
  for (int r = 0; r < nr; ++r) {
    const int64_t t = r0 + r;
    double v;
    if (kFp8In)
      v = (double)e4m3_to_f32(((const uint8_t*)q_in)[t * kIdxDim + j]) * (double)q_scale[t];
    else
      v = (double)((const float*)q_in)[t * kIdxDim + j];
    qrow[r][j] = v;
  }
  __syncthreads();

  double acc[kFoldRows];
#pragma unroll
  for (int r = 0; r < kFoldRows; ++r) acc[r] = 0.0;
  for (int i = 0; i < kIdxDim; ++i) {
    const double w = (double)wcol[i];
#pragma unroll
    for (int r = 0; r < kFoldRows; ++r) acc[r] = fma(qrow[r][i], w, acc[r]);
  }

  if (!kFp8In) {
    for (int r = 0; r < nr; ++r) ((float*)q_out)[(r0 + r) * kIdxDim + j] = (float)acc[r];
    return;
  }
  // per-row amax over the 128 columns (two waves)
  const int wv = j >> 6;
#pragma unroll
  for (int r = 0; r < kFoldRows; ++r) {
    double m = wave_max(fabs(acc[r]));
    if ((j & 63) == 0) wmax[wv][r] = m;
  }
  __syncthreads();
  for (int r = 0; r < nr; ++r) {
    const double amax = max(wmax[0][r], wmax[1][r]);
    const float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
    const uint32_t code = f64_to_e4m3_rne_sat(acc[r] / (double)s);
    ((uint8_t*)q_out)[(r0 + r) * kIdxDim + j] = (uint8_t)code;
    if (j == 0) s_out[r0 + r] = s;
  }
}

// Short batches (decode): the sum over i is split across four waves per
// column (32 terms each, in i order), and the four fp64 partials are added
// in a fixed order.  Two rows per block.
template <bool kFp8In, bool kWBf16>
__global__ __launch_bounds__(512) void fold_split_kernel(const void* __restrict__ q_in,
                                                         const float* __restrict__ q_scale,
                                                         const void* __restrict__ w_in, int64_t T,
                                                         void* __restrict__ q_out, float* __restrict__ s_out) {
  constexpr int R = 2, P = 4, IP = kIdxDim / P;
  __shared__ double qrow[R][kIdxDim];
  __shared__ double part[P][R][kIdxDim];
  __shared__ double wmax[2][R];
  const int tid = threadIdx.x, j = tid & (kIdxDim - 1), pi = tid / kIdxDim;
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int nr = (int)min<int64_t>(R, T - r0);
  if (tid < R * kIdxDim) {
    const int r = tid / kIdxDim;
    double v = 0.0;
    if (r < nr) {
      const int64_t t = r0 + r;
      if (kFp8In)
        v = (double)e4m3_to_f32(((const uint8_t*)q_in)[t * kIdxDim + j]) * (double)q_scale[t];
      else
        v = (double)((const float*)q_in)[t * kIdxDim + j];
    }
    qrow[r][j] = v;
  }
  float wcol[IP];
#pragma unroll
  for (int ii = 0; ii < IP; ++ii) {
    const int i = pi * IP + ii;
    if (kWBf16)
      wcol[ii] = bf16_to_f32(((const uint16_t*)w_in)[i * kIdxDim + j]);
    else
      wcol[ii] = ((const float*)w_in)[i * kIdxDim + j];
  }
  __syncthreads();
  double acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0;
#pragma unroll
  for (int ii = 0; ii < IP; ++ii) {
    const double w = (double)wcol[ii];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fma(qrow[r][pi * IP + ii], w, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) part[pi][r][j] = acc[r];
  __syncthreads();
  const bool own = tid < kIdxDim;
  double sum[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    sum[r] = own ? ((part[0][r][j] + part[1][r][j]) + part[2][r][j]) + part[3][r][j] : 0.0;
  if (!kFp8In) {
    if (own)
      for (int r = 0; r < nr; ++r) ((float*)q_out)[(r0 + r) * kIdxDim + j] = (float)sum[r];
    return;
  }
  // per-row amax over the 128 columns (waves 0 and 1)
  const int wv = tid >> 6;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double m = wave_max(fabs(sum[r]));
    if (wv < 2 && (tid & 63) == 0) wmax[wv][r] = m;
  }
  __syncthreads();
  if (!own) return;
  for (int r = 0; r < nr; ++r) {
    const double amax = max(wmax[0][r], wmax[1][r]);
    const float sc = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
    const uint32_t code = f64_to_e4m3_rne_sat(sum[r] / (double)sc);
    ((uint8_t*)q_out)[(r0 + r) * kIdxDim + j] = (uint8_t)code;
    if (j == 0) s_out[r0 + r] = sc;
  }
}

// Long prefills (FP8 input, bf16 W): tiles of TR rows (64, or 32 when 64-row
// tiles would leave CUs idle), 256 threads, each thread a register tile of
// TR/8 rows x 4 columns of fp64 accumulators, the rows' dequantised values as
// fp64 in LDS (k-major, so a thread's rows are one contiguous read) and W as
// fp32 in LDS (4 columns in one 16-byte read).  A block converts W once and
// walks tiles blockIdx.x, blockIdx.x + gridDim.x, ..., loading the next
// tile's codes while it computes the current one.  The per-row amax is a
// reduction over the 32 threads sharing the row.
template <int TR>
__global__ __launch_bounds__(256, 1) void fold_tile_kernel(const uint8_t* __restrict__ q_in,
                                                           const float* __restrict__ q_scale,
                                                           const uint16_t* __restrict__ w_in, int64_t T,
                                                           uint8_t* __restrict__ q_out, float* __restrict__ s_out) {
  constexpr int RPT = TR / 8;          // rows per thread
  constexpr int TPR = 256 / TR;        // threads loading one row's codes
  constexpr int CB = kIdxDim / TPR;    // code bytes per thread (32 or 16)
  static_assert(TR == 32 || TR == 64, "tile heights of 32 or 64 rows");
  extern __shared__ __align__(16) char fold_smem[];
  float* sw = (float*)fold_smem;                                    // [k][j], 64 KB
  double* sq = (double*)(fold_smem + kIdxDim * kIdxDim * 4);        // [k][row], 8 TR KB
  const int tid = threadIdx.x;
  const int tx = tid & 31, ty = tid >> 5;   // columns 4 tx .. +3, rows RPT ty .. +RPT-1
  const int lr = tid / TPR, lk = CB * (tid % TPR);  // the codes this thread loads: row lr, dims lk .. lk+CB-1
  const int64_t ntile = (T + TR - 1) / TR;
  {
    uint4 wb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wb[i] = ((const uint4*)w_in)[tid + 256 * i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 8 * (tid + 256 * i);
      const uint32_t u[4] = {wb[i].x, wb[i].y, wb[i].z, wb[i].w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
        *(float2*)(sw + e + 2 * h) = make_float2(__uint_as_float(u[h] << 16), __uint_as_float(u[h] & 0xFFFF0000u));
    }
  }
  auto load = [&](int64_t tile, uint4 (&codes)[CB / 16], float& scale) {
    const int64_t t = tile * TR + lr;
#pragma unroll
    for (int i = 0; i < CB / 16; ++i) codes[i] = make_uint4(0u, 0u, 0u, 0u);
    scale = 0.f;
    if (tile < ntile && t < T) {
#pragma unroll
      for (int i = 0; i < CB / 16; ++i) codes[i] = *(const uint4*)(q_in + t * kIdxDim + lk + 16 * i);
      scale = q_scale[t];
    }
  };
  uint4 codes[CB / 16];
  float scale;
  load(blockIdx.x, codes, scale);
  for (int64_t tile = blockIdx.x; tile < ntile; tile += gridDim.x) {
    __syncthreads();   // the previous tile's reads of sq are done
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const uint4 q4 = codes[j >> 4];
      const uint32_t wd = (j & 15) < 4 ? q4.x : (j & 15) < 8 ? q4.y : (j & 15) < 12 ? q4.z : q4.w;
      const uint32_t c = (wd >> (8 * (j & 3))) & 0xFFu;
      sq[(lk + j) * TR + lr] = (double)e4m3_to_f32(c) * (double)scale;
    }
    __syncthreads();
    load(tile + gridDim.x, codes, scale);
    double acc[RPT][4];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
    // the LDS reads of step k + 1 are issued before the FMAs of step k
    auto rd = [&](int k, float4& wv, double2 (&qv)[RPT / 2]) {
      wv = *(const float4*)(sw + k * kIdxDim + 4 * tx);
#pragma unroll
      for (int r = 0; r < RPT / 2; ++r) qv[r] = *(const double2*)(sq + k * TR + RPT * ty + 2 * r);
    };
    auto fmas = [&](const float4& wv, const double2 (&qv)[RPT / 2]) {
      const double w4[4] = {(double)wv.x, (double)wv.y, (double)wv.z, (double)wv.w};
#pragma unroll
      for (int r = 0; r < RPT / 2; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * r][c] = fma(qv[r].x, w4[c], acc[2 * r][c]);
          acc[2 * r + 1][c] = fma(qv[r].y, w4[c], acc[2 * r + 1][c]);
        }
    };
    float4 wa, wb;
    double2 qa[RPT / 2], qb[RPT / 2];
    rd(0, wa, qa);
    for (int k = 0; k < kIdxDim; k += 2) {
      rd(k + 1, wb, qb);
      fmas(wa, qa);
      if (k + 2 < kIdxDim) rd(k + 2, wa, qa);
      fmas(wb, qb);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int64_t t = tile * TR + RPT * ty + r;
      double m = fmax(fmax(fabs(acc[r][0]), fabs(acc[r][1])), fmax(fabs(acc[r][2]), fabs(acc[r][3])));
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
      const float sc = m > 0.0 ? (float)(m / 448.0) : 1.0f;
      if (t < T) {
        uint32_t pk = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) pk |= f64_to_e4m3_rne_sat(acc[r][c] / (double)sc) << (8 * c);
        *(uint32_t*)(q_out + t * kIdxDim + 4 * tx) = pk;
        if (tx == 0) s_out[t] = sc;
      }
    }
  }
}
constexpr size_t fold_tile_lds(int tr) { return (size_t)kIdxDim * kIdxDim * 4 + (size_t)kIdxDim * tr * 8; }

template <int R>
static void launch_fold_rows(const void* q_in, const float* q_scale, bool fp8_in, const void* w, bool w_bf16,
                             int64_t T, void* q_out, float* s_out, hipStream_t st) {
  dim3 grid((unsigned)((T + R - 1) / R));
  if (fp8_in && w_bf16)
    fold_kernel<true, true, R><<<grid, 128, 0, st>>>(q_in, q_scale, w, T, q_out, s_out);
  else if (fp8_in)
    fold_kernel<true, false, R><<<grid, 128, 0, st>>>(q_in, q_scale, w, T, q_out, s_out);
  else
    fold_kernel<false, false, R><<<grid, 128, 0, st>>>(q_in, q_scale, w, T, q_out, s_out);
}

hipError_t launch_fold(const void* q_in, const float* q_scale, bool fp8_in, const void* w,
                       bool w_bf16, int64_t T, void* q_out, float* s_out, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  // the tiled kernel's vector accesses: 32-byte code rows, 16-byte W reads,
  // 4-byte packed stores
  const bool tile_ok = ((uintptr_t)q_in % 32 == 0) && ((uintptr_t)w % 16 == 0) && ((uintptr_t)q_out % 4 == 0);
  if (T >= 8192 && fp8_in && w_bf16 && tile_ok) {
    int cus = 256;
    {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    }
    // 64-row tiles once they cover every CU, else 32-row tiles (twice the blocks)
    const int64_t tiles64 = (T + 63) / 64;
    if (tiles64 >= cus) {
      static std::atomic<uint64_t> lds_done{0};
      const hipError_t e = set_lds_limit_once((const void*)fold_tile_kernel<64>, (int)fold_tile_lds(64), lds_done);
      if (e != hipSuccess) return e;
      fold_tile_kernel<64><<<(unsigned)cus, 256, fold_tile_lds(64), st>>>(
          (const uint8_t*)q_in, q_scale, (const uint16_t*)w, T, (uint8_t*)q_out, s_out);
    } else {
      static std::atomic<uint64_t> lds_done{0};
      const hipError_t e = set_lds_limit_once((const void*)fold_tile_kernel<32>, (int)fold_tile_lds(32), lds_done);
      if (e != hipSuccess) return e;
      const int64_t tiles = (T + 31) / 32;
      fold_tile_kernel<32><<<(unsigned)(tiles < cus ? tiles : cus), 256, fold_tile_lds(32), st>>>(
          (const uint8_t*)q_in, q_scale, (const uint16_t*)w, T, (uint8_t*)q_out, s_out);
    }
  } else if (T >= 8192)
    launch_fold_rows<32>(q_in, q_scale, fp8_in, w, w_bf16, T, q_out, s_out, st);
  else {
    dim3 grid((unsigned)((T + 1) / 2));
    if (fp8_in && w_bf16)
      fold_split_kernel<true, true><<<grid, 512, 0, st>>>(q_in, q_scale, w, T, q_out, s_out);
    else if (fp8_in)
      fold_split_kernel<true, false><<<grid, 512, 0, st>>>(q_in, q_scale, w, T, q_out, s_out);
    else
      fold_split_kernel<false, false><<<grid, 512, 0, st>>>(q_in, q_scale, w, T, q_out, s_out);
  }
  return hipGetLastError();
}

}  // namespace dsa
