// Fold W_index into the index query and re-quantise it to e4m3.
//
// The indexer score is q_t . W_index . k_s (DeepSeek-V3.2 write-up, section
// 2.2).  Folding W into q once per query turns the per-pair work into one
// 128-wide FP8 dot product; the folded row is re-quantised with its own
// amax/448 scale so that the pair product stays FP8.
//
// Work: T x 128 x 128 MACs in fp64 (bit-reproducible codes), ~1/1024 of the
// indexer's pair work.  One thread owns one output column j and keeps column
// j of W in registers; a block walks kRows query rows held in LDS as fp64.
// Short batches split each column's sum over four waves instead.
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
  if (T >= 8192)
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
