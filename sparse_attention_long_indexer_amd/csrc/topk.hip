// Per-row top-k selection over materialised scores (DeepSeek-V3.2 write-up,
// section 2.3: keep the k best-scoring keys of each query).
//
// One 1024-thread block per row.  Scores map to order-preserving uint32 keys
// (larger score -> larger key, -0.0 folded onto +0.0).  A most-significant-
// digit-first radix select with four 8-bit digits finds the exact key of the
// m-th best element and how many elements equal to it are kept; LDS
// histograms take one atomic per element, except the key of a zero score,
// which ReLU makes the common tie and which is counted with a wave ballot.
// A last pass walks the row in index order with block-wide prefix counts
// (wave ballots + per-wave totals in LDS), keeps every key above the
// threshold and the lowest-index keys equal to it, and writes the kept
// indices in ascending order.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace dsa {


struct RowView {
  const float* p;
  int64_t n;
};

__device__ __forceinline__ RowView topk_row_view(const TopkRows& R, int64_t row) {
  RowView v;
  if (R.seq_offsets) {
    const int64_t lo = R.seq_offsets[row];
    v.p = R.scores + lo;
    v.n = R.seq_offsets[row + 1] - lo;
  } else {
    const int64_t t = R.row_begin + row;
    const int64_t pos = R.q_pos ? R.q_pos[t] : t;
    int64_t n = pos + 1 < R.S ? pos + 1 : R.S;
    v.n = n > 0 ? n : 0;
    v.p = R.scores + (R.row_off ? R.row_off[row] : row * R.ld);
  }
  return v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_radix_kernel(TopkRows R, int64_t k,
                                                                  int32_t* __restrict__ idx_out,
                                                                  int32_t* __restrict__ count_out) {
  __shared__ TopkShared sh;
  const int64_t row = blockIdx.x;
  const RowView rv = topk_row_view(R, row);
  if (count_out && threadIdx.x == 0) count_out[row] = (int32_t)(rv.n < k ? rv.n : k);
  select_row(rv.p, rv.n, k, idx_out + row * k, sh);
}

size_t topk_workspace_bytes(int64_t rows, int64_t max_n, int64_t k) {
  (void)rows;
  (void)max_n;
  (void)k;
  return 0;
}

hipError_t launch_topk(const TopkRows& r, int64_t rows, int64_t max_n, int64_t k, int32_t* idx_out,
                       int32_t* count_out, void* ws, hipStream_t st) {
  (void)max_n;
  (void)ws;
  if (rows <= 0) return hipSuccess;
  topk_radix_kernel<<<(unsigned)rows, kTopkThreads, 0, st>>>(r, k, idx_out, count_out);
  return hipGetLastError();
}

}  // namespace dsa
