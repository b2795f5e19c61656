// Host-side safety driver for the C ABI (include/m2rnn.h), built together
// with the library sources by tests/test_abi_sanitized.py with the host
// code under AddressSanitizer and UndefinedBehaviorSanitizer.  It needs no
// GPU: every call below fails argument validation, which the library
// finishes before any HIP call, and the workspace-size queries are host
// arithmetic.  Checked: each bad argument gets its documented status and a
// non-empty message, and the size queries neither overflow nor misbehave at
// the extremes of int (UBSan reports signed overflow).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "m2rnn.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  const char* msg = m2rnn_last_error();
  if (got != want || !msg || !msg[0]) {
    std::fprintf(stderr, "FAILED: %s: status %d (want %d), message \"%s\"\n", what, got, want, msg ? msg : "(null)");
    ++failures;
  }
}

int main() {
  alignas(256) static unsigned char buf[1 << 16];
  void* p = buf;                            // aligned, non-null
  float* pf = reinterpret_cast<float*>(buf);
  void* mis = buf + 2;                      // misaligned for every tensor
  float* misf = reinterpret_cast<float*>(buf + 2);
  const int F32 = M2RNN_F32, BF16 = M2RNN_BF16;

  // forward
  expect(m2rnn_forward(-1, 8, 4, 64, 16, F32, p, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr, 0, nullptr),
         M2RNN_ERR_INVALID_ARG, "forward B < 0");
  expect(m2rnn_forward(1, 8, 4, 32, 16, F32, p, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr, 0, nullptr),
         M2RNN_ERR_UNSUPPORTED, "forward K != 64");
  expect(m2rnn_forward(1, 8, 4, 64, 8, F32, p, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr, 0, nullptr),
         M2RNN_ERR_UNSUPPORTED, "forward V != 16");
  expect(m2rnn_forward(1, 8, 4, 64, 16, 7, p, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr, 0, nullptr),
         M2RNN_ERR_INVALID_ARG, "forward bad dtype");
  expect(m2rnn_forward(1, 8, 4, 64, 16, BF16, nullptr, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr, 0,
                       nullptr),
         M2RNN_ERR_INVALID_ARG, "forward q NULL");
  expect(m2rnn_forward(1, 8, 4, 64, 16, BF16, mis, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr, 0, nullptr),
         M2RNN_ERR_INVALID_ARG, "forward q misaligned");
  expect(m2rnn_forward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, misf, pf, pf, nullptr, 0, nullptr, 0, nullptr),
         M2RNN_ERR_INVALID_ARG, "forward H_0 misaligned");
  expect(m2rnn_forward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, nullptr, pf, pf, nullptr, -1, nullptr, 0, nullptr),
         M2RNN_ERR_INVALID_ARG, "forward ckpt_every < 0");
  expect(m2rnn_forward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, nullptr, pf, pf, pf, 0, nullptr, 0, nullptr),
         M2RNN_ERR_INVALID_ARG, "forward H_ckpt without ckpt_every");
  expect(m2rnn_forward(INT_MAX, INT_MAX, INT_MAX, 64, 16, F32, p, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr,
                       0, nullptr),
         M2RNN_ERR_UNSUPPORTED, "forward beyond the size limits");
  expect(m2rnn_forward_gated(1, 8, 4, 64, 16, F32, p, p, p, nullptr, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr,
                             0, nullptr),
         M2RNN_ERR_INVALID_ARG, "forward_gated a NULL");
  // the row-split path needs a workspace: a few chains, none given
  expect(m2rnn_forward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, nullptr, pf, pf, nullptr, 0, nullptr, 0, nullptr),
         M2RNN_ERR_WORKSPACE, "forward without its workspace");

  // backward
  expect(m2rnn_backward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, pf, 0, pf, nullptr, pf, pf, pf, pf, pf, pf, nullptr,
                        p, sizeof buf, nullptr),
         M2RNN_ERR_INVALID_ARG, "backward ckpt_every 0");
  expect(m2rnn_backward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, nullptr, 4, pf, nullptr, pf, pf, pf, pf, pf, pf,
                        nullptr, p, sizeof buf, nullptr),
         M2RNN_ERR_INVALID_ARG, "backward H_ckpt NULL");
  expect(m2rnn_backward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, pf, 4, pf, misf, pf, pf, pf, pf, pf, pf, nullptr, p,
                        sizeof buf, nullptr),
         M2RNN_ERR_INVALID_ARG, "backward dH_T misaligned");
  expect(m2rnn_backward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, pf, 4, pf, nullptr, pf, pf, pf, pf, pf, pf, nullptr,
                        p, 16, nullptr),
         M2RNN_ERR_WORKSPACE, "backward workspace too small");
  expect(m2rnn_backward(1, 8, 4, 64, 16, F32, p, p, p, p, p, p, pf, 4, pf, nullptr, pf, pf, pf, pf, pf, pf, nullptr,
                        mis, sizeof buf, nullptr),
         M2RNN_ERR_INVALID_ARG, "backward workspace misaligned");
  expect(m2rnn_backward_gated(1, 8, 4, 64, 16, F32, p, p, p, p, nullptr, p, p, p, pf, 4, pf, nullptr, pf, pf, pf, pf,
                              pf, pf, pf, pf, nullptr, p, sizeof buf, nullptr),
         M2RNN_ERR_INVALID_ARG, "backward_gated alpha NULL");

  // epilogue, prologue, decode
  expect(m2rnn_gate_rmsnorm_forward(1, 8, 4, 16, F32, pf, p, p, -1.0f, pf, nullptr, nullptr), M2RNN_ERR_INVALID_ARG,
         "rmsnorm eps < 0");
  expect(m2rnn_gate_rmsnorm_forward(1, 8, 3, 5, F32, pf, p, p, 1e-6f, pf, nullptr, nullptr), M2RNN_ERR_UNSUPPORTED,
         "rmsnorm N V not a multiple of 4");
  expect(m2rnn_gate_rmsnorm_backward(1, 8, 4, 16, F32, pf, p, p, 1e-6f, pf, pf, pf, pf, nullptr, 0, nullptr),
         M2RNN_ERR_WORKSPACE, "rmsnorm backward without its workspace");
  expect(m2rnn_gate_rmsnorm_backward_noalloc(1, 8, 4, 16, 9, pf, p, p, 1e-6f, pf, pf, pf, pf, nullptr),
         M2RNN_ERR_INVALID_ARG, "rmsnorm backward (no allocation) bad dtype");
  expect(m2rnn_conv_silu_forward(1, 8, 6, F32, p, p, nullptr, p, nullptr), M2RNN_ERR_UNSUPPORTED,
         "conv C not a multiple of 4");
  expect(m2rnn_conv_silu_backward(1, 8, 8, F32, p, p, nullptr, pf, nullptr, pf, nullptr, p, sizeof buf, nullptr),
         M2RNN_ERR_INVALID_ARG, "conv backward du NULL");
  expect(m2rnn_decode(2, 4, 64, 16, F32, p, p, p, p, p, p, nullptr, pf, nullptr), M2RNN_ERR_INVALID_ARG,
         "decode H NULL");

  // workspace sizes at the extremes of int: defined results, no overflow
  const int ext[] = {0, 1, 3, 64, 4096, 1 << 20, INT_MAX - 1, INT_MAX};
  size_t acc = 0;
  for (int B : ext)
    for (int T : ext)
      for (int N : ext) {
        acc += m2rnn_forward_workspace_bytes(B, T, N, 64, 16);
        acc += m2rnn_backward_workspace_bytes(B, T, N, 64, 16, 64);
        acc += m2rnn_backward_workspace_bytes(B, T, N, 64, 16, 1);
        acc += m2rnn_conv_silu_backward_workspace_bytes(B, T, N);
        acc += m2rnn_gate_rmsnorm_backward_workspace_bytes(B, T, N, 16);
      }
  acc += m2rnn_backward_workspace_bytes(1, 8, 4, 64, 16, 0) + m2rnn_backward_workspace_bytes(1, 8, 4, 64, 16, -5);
  acc += m2rnn_forward_workspace_bytes(-1, 8, 4, 64, 16) + m2rnn_gate_rmsnorm_backward_workspace_bytes(-1, -1, -1, -1);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("C ABI sanitizer driver: all calls clean (size checksum %zu)\n", acc);
  return 0;
}
