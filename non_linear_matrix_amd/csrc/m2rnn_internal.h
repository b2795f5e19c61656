// m2rnn_internal.h -- launch arguments shared by the C-ABI layer and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace m2rnn {

struct FwdArgs {
  const void *q, *k, *v, *f, *W, *wr;
  float *y, *H_T, *H_ckpt;
  int B, T, N;
  int ckpt_every;  // > 0 when H_ckpt != nullptr
  int nck;         // ceil(T / ckpt_every)
};

hipError_t launch_forward(const FwdArgs& a, int dtype, hipStream_t stream);

// Zero `n` floats with a plain fill kernel (graph-capture friendly).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream);

}  // namespace m2rnn
