// mx_pack_weights: e4m3 expert weights, row-major [E, N, Kd], into the
// tile-packed layout the *_packed GEMMs read.  It is this library's
// counterpart of the weight-format cast of the pages (weights cast once, at
// load time, into the matrix unit's tiled format: "PR #30768 report",
// review highlights on the NZ format; "[WIP] Fix offline W8A8 MXFP8
// quantization for Qwen3.5 on Ascend NPU", the commit on the NZ cast),
// shaped by what the GEMMs' LDS ring holds instead of by another chip's
// matrix unit.
//
// Layout.  For expert e, n-tile nt (256 weight rows) and k stage ks (128
// bytes of K), one 32 KB block at byte ((e * NT + nt) * (Kd / 128) + ks) *
// 32768 (NT = N / 256) holds the 256 rows in the order a GEMM workgroup's
// ring slot keeps them, 128 bytes each, with 16-byte chunk c of slot row r
// stored at chunk position c ^ ((r / 2) % 8), the slot's bank swizzle.  A
// stage's weight DMA is then one contiguous 32 KB read, every 1 KB
// instruction landing unchanged in LDS.  Slot row order, kind 0 (GEMM2,
// plain): slot row r is weight row 256 nt + r.  Kind 1 (GEMM1, N = 2I rows,
// gate rows [0, I) then up rows [I, 2I)): slot rows [128 h, 128 h + 64) are
// gate rows 128 nt + 64 h + (0..63) and slot rows [128 h + 64, 128 h + 128)
// the up rows I + 128 nt + 64 h + (0..63), h = 0, 1, so the gate and up rows
// of the same 128 h-columns share a block.  Scales keep their own layout.
#include "common.h"

namespace mxmoe {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void pack_weights_kernel(const uint8_t* __restrict__ w, int64_t E,
                                                                int64_t N, int64_t Kd, int kind,
                                                                uint8_t* __restrict__ out) {
  const int64_t nk = Kd / 128, NT = N / 256, I = N / 2;
  const int64_t total = E * N * (Kd / 16);   // 16-byte output chunks
  for (int64_t j = blockIdx.x * (int64_t)kThreads + threadIdx.x; j < total; j += (int64_t)gridDim.x * kThreads) {
    const int pc = (int)(j & 7);
    const int r = (int)((j >> 3) & 255);
    const int64_t blk = j >> 11;                // 2048 chunks = 32 KB per block
    const int64_t ks = blk % nk, rest = blk / nk;
    const int64_t nt = rest % NT, e = rest / NT;
    int64_t n;
    if (kind == 0) {
      n = nt * 256 + r;
    } else {
      const int h = r >> 7, rr = r & 127;
      n = (rr < 64 ? 0 : I) + nt * 128 + 64 * h + (rr & 63);
    }
    const int c = pc ^ ((r >> 1) & 7);         // logical chunk stored at position pc
    const uint4 v = *reinterpret_cast<const uint4*>(w + (e * N + n) * Kd + ks * 128 + c * 16);
    *reinterpret_cast<uint4*>(out + j * 16) = v;
  }
}

}  // namespace

}  // namespace mxmoe

extern "C" int mx_pack_weights(const void* w_u8, int64_t E, int64_t N, int64_t Kd, int kind, void* out_u8,
                               void* stream) {
  using namespace mxmoe;
  if (!w_u8 || !out_u8) return fail(MX_ERR_INVALID_ARG, "mx_pack_weights: null pointer");
  if (E <= 0 || N <= 0 || Kd <= 0)
    return fail(MX_ERR_INVALID_ARG, "mx_pack_weights: bad sizes E=%lld N=%lld Kd=%lld", (long long)E, (long long)N,
                (long long)Kd);
  if (kind != 0 && kind != 1)
    return fail(MX_ERR_INVALID_ARG, "mx_pack_weights: kind must be 0 (GEMM2 rows) or 1 (GEMM1 gate/up rows), got %d",
                kind);
  if (!dims_in_range({E, N, Kd}) || E > 1024 || Kd > ((int64_t)1 << 20))
    return fail(MX_ERR_UNSUPPORTED, "mx_pack_weights: E=%lld (max 1024), N=%lld or Kd=%lld (max 2^20) too large",
                (long long)E, (long long)N, (long long)Kd);
  if (N % 256 != 0 || Kd % 128 != 0)
    return fail(MX_ERR_UNSUPPORTED, "mx_pack_weights: N=%lld must be a multiple of 256 and Kd=%lld of 128",
                (long long)N, (long long)Kd);
  if (reinterpret_cast<uintptr_t>(w_u8) % 16 || reinterpret_cast<uintptr_t>(out_u8) % 16)
    return fail(MX_ERR_UNSUPPORTED, "mx_pack_weights: w and out must be 16-byte aligned");
  const uintptr_t bytes = (uintptr_t)(E * N) * (uintptr_t)Kd;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w_u8), b = reinterpret_cast<uintptr_t>(out_u8);
  if (a < b + bytes && b < a + bytes) return fail(MX_ERR_INVALID_ARG, "mx_pack_weights: w and out overlap");
  const int64_t total = E * N * (Kd / 16);
  int64_t grid = (total + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)num_cus() * 16;
  if (grid > cap) grid = cap;
  pack_weights_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, as_stream(stream)>>>(
      static_cast<const uint8_t*>(w_u8), E, N, Kd, kind, static_cast<uint8_t*>(out_u8));
  return check_launch("mx_pack_weights");
}
