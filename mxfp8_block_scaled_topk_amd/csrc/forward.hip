// moe_mxfp8_forward: the whole expert layer on one stream.
//
//   moe_route_quant -> gmm_swiglu_mxquant -> gmm_mx -> moe_finalize
//
// All intermediates live in one caller-provided workspace; the per-expert
// row counts stay on the device (the GEMMs read them directly), so the host
// never waits on the GPU.
#include "common.h"

namespace mxmoe {

int check_route_args(int64_t T, int64_t K, int64_t k, int64_t E);
size_t route_workspace_bytes(int64_t T, int64_t k, int64_t E);
int launch_route_quant(const uint16_t* x, const int32_t* ids, int64_t T, int64_t K, int64_t k, int64_t E,
                       uint8_t* xq, uint8_t* xs, int32_t* sorted_row, int32_t* eri, int64_t* group_list,
                       void* ws, hipStream_t stream);
int check_gmm_common(const char* name, int gl_type, int64_t M, int64_t Kd, int64_t E);
int launch_gmm_swiglu(const uint8_t* a, const uint8_t* as, const uint8_t* w13, const uint8_t* w13s,
                      const int64_t* gl, int gl_type, int64_t M, int64_t K, int64_t I, int64_t E, uint8_t* hq,
                      uint8_t* hs, float* hdbg, hipStream_t stream, int wf);
int launch_gmm_mx(const uint8_t* a, const uint8_t* as, const uint8_t* w, const uint8_t* ws, const int64_t* gl,
                  int gl_type, int64_t M, int64_t N, int64_t Kd, int64_t E, uint16_t* y, hipStream_t stream,
                  int wf);
int launch_finalize(const uint16_t* y, const float* w, const int32_t* eri, int64_t T, int64_t K, int64_t k,
                    int64_t M, uint16_t* out, hipStream_t stream);

namespace {

struct Layout {
  size_t off[9];   // xq, xs, sorted_row, eri, group_list, hq, hs, y, route workspace
  size_t total;
};

Layout layout(int64_t T, int64_t K, int64_t I, int64_t E, int64_t k) {
  const size_t M = (size_t)(T * k);
  const size_t sizes[9] = {
      M * (size_t)K,                       // xq
      M * (size_t)((K / 64) * 2),          // xs
      M * 4,                               // sorted_row
      M * 4,                               // expanded_row_idx
      (size_t)E * 8,                       // group_list
      M * (size_t)I,                       // hq
      M * (size_t)(I / 32),                // hs
      M * (size_t)K * 2,                   // y
      route_workspace_bytes(T, k, E),      // routing scratch
  };
  Layout L{};
  size_t cur = 0;
  for (int i = 0; i < 9; ++i) {
    L.off[i] = cur;
    cur += align_up(sizes[i], 256);
  }
  L.total = cur;
  return L;
}

int check_forward_args(int64_t T, int64_t K, int64_t I, int64_t E, int64_t k) {
  int rc = check_route_args(T, K, k, E);
  if (rc) return rc;
  if (I <= 0) return fail(MX_ERR_INVALID_ARG, "moe_mxfp8_forward: bad I=%lld", (long long)I);
  if (!dims_in_range({I})) return fail(MX_ERR_UNSUPPORTED, "moe_mxfp8_forward: I above 2^31 - 1");
  if (K % 256 != 0 || I % 128 != 0)
    return fail(MX_ERR_UNSUPPORTED, "moe_mxfp8_forward: K=%lld must be a multiple of 256 and I=%lld of 128",
                (long long)K, (long long)I);
  return check_gmm_common("moe_mxfp8_forward", 1, T * k, K, E);
}

}  // namespace

}  // namespace mxmoe

extern "C" size_t moe_mxfp8_forward_workspace_size(int64_t T, int64_t K, int64_t I, int64_t E, int64_t k) {
  // 0 for sizes the forward rejects
  if (mxmoe::check_forward_args(T, K, I, E, k) != MX_OK) return 0;
  return mxmoe::layout(T, K, I, E, k).total;
}

extern "C" int moe_mxfp8_forward_workspace_layout(int64_t T, int64_t K, int64_t I, int64_t E, int64_t k,
                                                  size_t* offsets_host) {
  using namespace mxmoe;
  int rc = check_forward_args(T, K, I, E, k);
  if (rc) return rc;
  if (!offsets_host) return fail(MX_ERR_INVALID_ARG, "moe_mxfp8_forward_workspace_layout: null pointer");
  const Layout L = layout(T, K, I, E, k);
  for (int i = 0; i < 8; ++i) offsets_host[i] = L.off[i];
  return MX_OK;
}

namespace {

// The layer on one stream; wf: the expert weights' format (e4m3 rows, MXFP4
// packed e2m1 for the W4A8 path, or e4m3 tile-packed by mx_pack_weights);
// the activations are MXFP8 either way.
int forward(const char* name, int wf, const void* x_bf16, const int32_t* topk_ids, const float* topk_w,
            const void* w13_u8, const void* w13_s, const void* w2_u8, const void* w2_s, int64_t T, int64_t K,
            int64_t I, int64_t E, int64_t k, void* out_bf16, void* workspace, size_t ws_bytes, void* stream) {
  using namespace mxmoe;
  int rc = check_forward_args(T, K, I, E, k);
  if (rc) return rc;
  if (!workspace) return fail(MX_ERR_INVALID_ARG, "%s: null workspace", name);
  if (T > 0 && (!x_bf16 || !topk_ids || !topk_w || !w13_u8 || !w13_s || !w2_u8 || !w2_s || !out_bf16))
    return fail(MX_ERR_INVALID_ARG, "%s: null pointer", name);
  const Layout L = layout(T, K, I, E, k);
  if (ws_bytes < L.total)
    return fail(MX_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", name, ws_bytes, L.total);
  const uintptr_t align_or = reinterpret_cast<uintptr_t>(x_bf16) | reinterpret_cast<uintptr_t>(w13_u8) |
                             reinterpret_cast<uintptr_t>(w2_u8) | reinterpret_cast<uintptr_t>(out_bf16) |
                             reinterpret_cast<uintptr_t>(workspace);
  const uintptr_t align_s = reinterpret_cast<uintptr_t>(w13_s) | reinterpret_cast<uintptr_t>(w2_s);
  if (align_or % 16 || align_s % 4)
    return fail(MX_ERR_UNSUPPORTED, "%s: misaligned pointer", name);
  if (T == 0) return MX_OK;
  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.off[0]);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + L.off[1]);
  int32_t* sorted_row = reinterpret_cast<int32_t*>(ws + L.off[2]);
  int32_t* eri = reinterpret_cast<int32_t*>(ws + L.off[3]);
  int64_t* gl = reinterpret_cast<int64_t*>(ws + L.off[4]);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.off[5]);
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + L.off[6]);
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.off[7]);
  void* rws = ws + L.off[8];
  const int64_t M = T * k;
  rc = launch_route_quant(static_cast<const uint16_t*>(x_bf16), topk_ids, T, K, k, E, xq, xs, sorted_row, eri, gl,
                          rws, s);
  if (rc) return rc;
  rc = launch_gmm_swiglu(xq, xs, static_cast<const uint8_t*>(w13_u8), static_cast<const uint8_t*>(w13_s), gl, 1, M,
                         K, I, E, hq, hs, nullptr, s, wf);
  if (rc) return rc;
  rc = launch_gmm_mx(hq, hs, static_cast<const uint8_t*>(w2_u8), static_cast<const uint8_t*>(w2_s), gl, 1, M, K, I,
                     E, y, s, wf);
  if (rc) return rc;
  return launch_finalize(y, topk_w, eri, T, K, k, M, static_cast<uint16_t*>(out_bf16), s);
}

}  // namespace

extern "C" int moe_mxfp8_forward(const void* x_bf16, const int32_t* topk_ids, const float* topk_w,
                                 const void* w13_u8, const void* w13_s, const void* w2_u8, const void* w2_s,
                                 int64_t T, int64_t K, int64_t I, int64_t E, int64_t k, void* out_bf16,
                                 void* workspace, size_t ws_bytes, void* stream) {
  return forward("moe_mxfp8_forward", mxmoe::kWfE4m3, x_bf16, topk_ids, topk_w, w13_u8, w13_s, w2_u8, w2_s, T, K, I, E, k,
                 out_bf16, workspace, ws_bytes, stream);
}

extern "C" int moe_w4a8_forward(const void* x_bf16, const int32_t* topk_ids, const float* topk_w,
                                const void* w13_u8, const void* w13_s, const void* w2_u8, const void* w2_s,
                                int64_t T, int64_t K, int64_t I, int64_t E, int64_t k, void* out_bf16,
                                void* workspace, size_t ws_bytes, void* stream) {
  return forward("moe_w4a8_forward", mxmoe::kWfE2m1, x_bf16, topk_ids, topk_w, w13_u8, w13_s, w2_u8, w2_s, T, K, I, E, k,
                 out_bf16, workspace, ws_bytes, stream);
}

extern "C" int moe_mxfp8_forward_packed(const void* x_bf16, const int32_t* topk_ids, const float* topk_w,
                                        const void* w13_packed, const void* w13_s, const void* w2_packed,
                                        const void* w2_s, int64_t T, int64_t K, int64_t I, int64_t E, int64_t k,
                                        void* out_bf16, void* workspace, size_t ws_bytes, void* stream) {
  return forward("moe_mxfp8_forward_packed", mxmoe::kWfPacked, x_bf16, topk_ids, topk_w, w13_packed, w13_s,
                 w2_packed, w2_s, T, K, I, E, k, out_bf16, workspace, ws_bytes, stream);
}
