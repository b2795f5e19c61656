// m2rnn_colsum.hip -- deterministic column sums of per-worker partials.
//
// out[col] = sum over rows of in[row][col], in two fixed-order levels so that
// many loads are in flight: block (cx, ry) of kColsumRowBlocks row blocks has
// 64 f4 columns x 4 row lanes; lane r sums rows ry 4 + r + k 4 R (k ascending,
// four interleaved accumulators), the four lanes are added in order into
// ws2[ry][cols]; then each column adds its R values in order.
#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {

namespace {

__global__ __launch_bounds__(256) void colsum_partial_kernel(const float* in, int rows, int cols, float* ws2) {
  __shared__ f4 lanes[4][64];
  const int col = blockIdx.x * 64 + threadIdx.x % 64, r = threadIdx.x / 64, ry = blockIdx.y;
  const int c4 = cols / 4;
  f4 acc[4] = {};
  if (col < c4) {
    const int stride = 4 * kColsumRowBlocks;
    int row = ry * 4 + r;
    for (; row + 3 * stride < rows; row += 4 * stride) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += *(const f4*)(in + (size_t)(row + q * stride) * cols + col * 4);
    }
    for (int q = 0; row < rows; row += stride, ++q) acc[q] += *(const f4*)(in + (size_t)row * cols + col * 4);
  }
  lanes[r][threadIdx.x % 64] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (r == 0 && col < c4) {
    const int c = threadIdx.x % 64;
    *(f4*)(ws2 + (size_t)ry * cols + col * 4) = (lanes[0][c] + lanes[1][c]) + (lanes[2][c] + lanes[3][c]);
  }
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float* ws2, int cols, float* out_a, int cols_a,
                                                           float* out_b) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= cols / 4) return;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int ry = 0; ry < kColsumRowBlocks; ++ry) acc += *(const f4*)(ws2 + (size_t)ry * cols + col * 4);
  if (col * 4 < cols_a) *(f4*)(out_a + col * 4) = acc;
  else if (out_b) *(f4*)(out_b + (col * 4 - cols_a)) = acc;
}

}  // namespace

hipError_t launch_colsum(const float* in, int rows, int cols, float* ws2, float* out_a, int cols_a, float* out_b,
                         hipStream_t stream) {
  const dim3 pgrid((unsigned)((cols / 4 + 63) / 64), (unsigned)kColsumRowBlocks);
  hipLaunchKernelGGL(colsum_partial_kernel, pgrid, dim3(256), 0, stream, in, rows, cols, ws2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((cols / 4 + 255) / 256)), dim3(256), 0, stream, ws2, cols,
                     out_a, cols_a, out_b);
  return hipGetLastError();
}

}  // namespace m2rnn
