// mx_linear: a dense MXFP8 linear layer ("Quantization on Ascend", MXFP8
// (dense) implementation notes: weights MX-quantised once at load,
// activations MX-quantised per token at inference, block 32 along K, then
// the quantised matmul).
//
//   (xq, xs) = MX quantisation of x [T, K] along K        (mx_quantize)
//   y [T, N] = bf16( sum over blocks 2^(sx + sw) * (xq . wq) )   (gmm_mx, one group)
//
// The GEMM is the grouped block-scaled MFMA GEMM with a single group of T
// rows (group-list type 2 inside the library: no list in memory).
#include "common.h"

namespace mxmoe {

int launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t kd, int64_t ld, uint8_t* q, uint8_t* s,
                       hipStream_t stream);
int check_gmm_common(const char* name, int gl_type, int64_t M, int64_t Kd, int64_t E);
int launch_gmm_mx(const uint8_t* a, const uint8_t* as, const uint8_t* w, const uint8_t* ws, const int64_t* gl,
                  int gl_type, int64_t M, int64_t N, int64_t Kd, int64_t E, uint16_t* y, hipStream_t stream,
                  int wf);

namespace {

struct LinearLayout {
  size_t xq, xs, total;
};
LinearLayout linear_layout(int64_t T, int64_t K) {
  LinearLayout L;
  L.xq = 0;
  L.xs = align_up((size_t)(T * K), 256);
  L.total = L.xs + align_up((size_t)(T * (K / 32)), 256);
  return L;
}

}  // namespace

}  // namespace mxmoe

extern "C" size_t mx_linear_workspace_size(int64_t T, int64_t K) {
  // 0 for sizes mx_linear rejects
  if (mxmoe::check_gmm_common("mx_linear", 1, T, K, 1) != MX_OK) return 0;
  return mxmoe::linear_layout(T, K).total;
}

extern "C" int mx_linear(const void* x_bf16, const void* w_u8, const void* w_s, int64_t T, int64_t K, int64_t N,
                         void* y_bf16, void* workspace, size_t ws_bytes, void* stream) {
  using namespace mxmoe;
  int rc = check_gmm_common("mx_linear", 1, T, K, 1);
  if (rc) return rc;
  if (N <= 0) return fail(MX_ERR_INVALID_ARG, "mx_linear: bad N=%lld", (long long)N);
  if (!dims_in_range({N})) return fail(MX_ERR_UNSUPPORTED, "mx_linear: N above 2^31 - 1");
  if (N % 256 != 0) return fail(MX_ERR_UNSUPPORTED, "mx_linear: N=%lld is not a multiple of 256", (long long)N);
  if (T > 0 && (!x_bf16 || !w_u8 || !w_s || !y_bf16 || !workspace))
    return fail(MX_ERR_INVALID_ARG, "mx_linear: null pointer");
  const LinearLayout L = linear_layout(T, K);
  if (ws_bytes < L.total)
    return fail(MX_ERR_WORKSPACE, "mx_linear: workspace %zu bytes < %zu", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(x_bf16) % 16 || reinterpret_cast<uintptr_t>(w_u8) % 16 ||
      reinterpret_cast<uintptr_t>(w_s) % 4 || reinterpret_cast<uintptr_t>(y_bf16) % 16 ||
      reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(MX_ERR_UNSUPPORTED, "mx_linear: misaligned pointer");
  if (T == 0) return MX_OK;
  hipStream_t s = as_stream(stream);
  char* base = static_cast<char*>(workspace);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + L.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(base + L.xs);
  rc = launch_mx_quantize(static_cast<const uint16_t*>(x_bf16), T, K, K, xq, xs, s);
  if (rc) return rc;
  return launch_gmm_mx(xq, xs, static_cast<const uint8_t*>(w_u8), static_cast<const uint8_t*>(w_s), nullptr,
                       /*single group of T rows*/ 2, T, N, K, 1, static_cast<uint16_t*>(y_bf16), s, kWfE4m3);
}
