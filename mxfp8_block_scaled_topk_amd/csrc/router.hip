// moe_router: top-k softmax routing over a bf16 gate linear, upstream of the
// layer ("Quantization on Ascend", MXFP8 for LLM MoE models, implementation
// notes: the router gate is a plain linear layer, kept in bf16 on the online
// path).  For each token t:
//
//   logits[e] = sum_c x[t,c] * Wg[e,c]  (+ bias[e])       fp32 accumulation
//   p = softmax(logits over the E experts)
//   ids = the k largest logits, descending (equal logits: lower id first)
//   w[j] = p[ids[j]], divided by the sum of the k when renormalising
//
// One workgroup of 4 waves handles 64 tokens.  The gate GEMM runs on the bf16
// MFMA (V_MFMA_F32_32X32X16_BF16: lane l holds operand row l % 32 and the 8
// k-values [8 (l/32), 8 (l/32) + 8) of the 16-wide step; output lane l holds
// column l % 32 and rows 8 q + 4 (l/32) + (0..3) in accumulator elements
// 4 q .. 4 q + 3).  Gate rows are the A operand (experts), token rows the B
// operand.  K advances 64 values (128 bytes per row) per chunk through a
// double-buffered LDS tile of the 64 token rows and the E gate rows, loaded
// with 16-byte coalesced loads that run four chunks ahead through a ring of
// register sets (measured: with one chunk ahead the kernel waited out a
// memory round trip per chunk); 16-byte chunk c of row r sits at chunk
// c ^ (r % 8), which keeps the fragment reads (32 rows, one chunk) spread
// over the LDS banks.  Wave w covers tokens 32 (w % 2) .. + 32 and expert
// tiles w / 2, w / 2 + 2, ...  The logits then go through LDS to a quad of
// 4 lanes per token for the softmax and the selection (measured: one thread
// per token walking its row in LDS took two thirds of the kernel's time).  HBM-bound: x is read once
// (2 T K bytes), the gate comes from L2.
#include "common.h"

namespace mxmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kBT = 64;        // tokens per workgroup
constexpr int kCK = 64;        // k values per chunk (128 bytes of a row)
constexpr int kMaxE = 256;
constexpr int kRow = kCK * 2;  // bytes per row per chunk

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Buf {
  uint8_t x[kBT * kRow];     // 8 KB
  uint8_t g[kMaxE * kRow];   // 32 KB
};

// byte offset of 16-byte chunk c of row r in a tile of 128-byte rows
__device__ __forceinline__ int swz(int r, int c) { return r * kRow + ((c ^ (r & 7)) << 4); }

constexpr int kNone = 0x7fffffff;   // "no expert" in the top-k reductions

// Exchange with the lane whose index differs in bit 0 / bit 1 (within a quad).
template <int kCtrl>
__device__ __forceinline__ int quad_swap(int x) {
  return __builtin_amdgcn_update_dpp(x, x, kCtrl, 0xf, 0xf, false);
}
constexpr int kQuadXor1 = 0xb1;   // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4e;   // quad_perm [2, 3, 0, 1]
__device__ __forceinline__ float quad_swapf1(float x) {
  return __int_as_float(quad_swap<kQuadXor1>(__float_as_int(x)));
}
__device__ __forceinline__ float quad_swapf2(float x) {
  return __int_as_float(quad_swap<kQuadXor2>(__float_as_int(x)));
}
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, quad_swapf1(x));
  return fmaxf(x, quad_swapf2(x));
}
__device__ __forceinline__ float quad_sum(float x) {
  x += quad_swapf1(x);
  return x + quad_swapf2(x);
}
// (bv, be) <- the quad's largest bv, the lowest be among equal ones; lanes
// with be == kNone hold no candidate.
__device__ __forceinline__ void quad_argmax(float& bv, int& be) {
  auto take = [&](float ov, int oe) {
    if (oe != kNone && (be == kNone || ov > bv || (ov == bv && oe < be))) {
      bv = ov;
      be = oe;
    }
  };
  {
    const float ov = quad_swapf1(bv);
    const int oe = quad_swap<kQuadXor1>(be);
    take(ov, oe);
  }
  {
    const float ov = quad_swapf2(bv);
    const int oe = quad_swap<kQuadXor2>(be);
    take(ov, oe);
  }
}

template <int NT>   // expert tiles per wave (ceil(E/32) / 2, rounded up)
__global__ __launch_bounds__(kThreads) void router_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gate,
                                                          const float* __restrict__ bias, int64_t T, int64_t K,
                                                          int E, int k, int renormalize,
                                                          int32_t* __restrict__ topk_ids,
                                                          float* __restrict__ topk_w) {
  __shared__ __attribute__((aligned(16))) Buf buf[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kBT;
  const int Ep = (E + 31) & ~31;   // expert rows held in LDS
  const int nchunks = (int)(K / kCK);

  // ---- global -> registers -> LDS, one chunk ---------------------------------
  // x: 64 rows x 8 chunks, 2 per thread; gate: 64 NT rows (>= Ep) x 8 chunks,
  // 2 NT per thread.  Rows past T or E repeat the last row (their logits are
  // never selected or stored), so every thread issues the same loads.
  constexpr int kGPer = 2 * NT * 32 * 8 / kThreads;
  struct Regs {
    u32x4 x[2], g[kGPer];
  };
  auto load = [&](Regs& R, int ch) __attribute__((always_inline)) {
    u32x4(&rx)[2] = R.x;
    u32x4(&rg)[kGPer] = R.g;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + i * kThreads, r = piece >> 3, c = piece & 7;
      const int64_t row = t0 + r < T ? t0 + r : T - 1;
      rx[i] = *reinterpret_cast<const u32x4*>(x + row * K + (int64_t)ch * kCK + c * 8);
    }
#pragma unroll
    for (int i = 0; i < kGPer; ++i) {
      const int piece = tid + i * kThreads, r = piece >> 3, c = piece & 7;
      const int row = r < E ? r : E - 1;
      rg[i] = *reinterpret_cast<const u32x4*>(gate + (int64_t)row * K + (int64_t)ch * kCK + c * 8);
    }
  };
  auto store = [&](const Regs& R, Buf& b) __attribute__((always_inline)) {
    const u32x4(&rx)[2] = R.x;
    const u32x4(&rg)[kGPer] = R.g;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = tid + i * kThreads, r = piece >> 3, c = piece & 7;
      *reinterpret_cast<u32x4*>(b.x + swz(r, c)) = rx[i];
    }
#pragma unroll
    for (int i = 0; i < kGPer; ++i) {
      const int piece = tid + i * kThreads, r = piece >> 3, c = piece & 7;
      *reinterpret_cast<u32x4*>(b.g + swz(r, c)) = rg[i];
    }
  };

  const int th = wave & 1, eh = wave >> 1;
  const int li = lane & 31, lg = lane >> 5;
  v16f acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  // A ring of kDepth register sets: while chunk ch is multiplied, chunks
  // ch+1 .. ch+kDepth-1 are in flight or waiting in registers, and chunk
  // ch+kDepth is requested (one memory round trip per ~3 chunks of work).
  auto mfma_chunk = [&](const Buf& b) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kCK / 16; ++s) {
      const int c = 2 * s + lg;   // this lane's 16-byte chunk of the step
      const bf16x8 xb = *reinterpret_cast<const bf16x8*>(b.x + swz(32 * th + li, c));
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int et = eh + 2 * i;
        if (32 * et < Ep) {
          const bf16x8 gb = *reinterpret_cast<const bf16x8*>(b.g + swz(32 * et + li, c));
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gb, xb, acc[i], 0, 0, 0);
        }
      }
    }
  };
  // one step: multiply chunk ch (in buf[ch&1]), load chunk ch+kDepth into
  // `next` (it held chunk ch, already in LDS), move chunk ch+1 from `held`
  // into the other buffer
  constexpr int kDepth = 4;
  auto step = [&](int ch, Regs& held, Regs& next) __attribute__((always_inline)) {
    if (ch + kDepth < nchunks) load(next, ch + kDepth);
    mfma_chunk(buf[ch & 1]);
    if (ch + 1 < nchunks) store(held, buf[(ch + 1) & 1]);
    __syncthreads();
  };
  Regs R[kDepth];
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (j < nchunks) load(R[j], j);
  store(R[0], buf[0]);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ch += kDepth) {
    step(ch, R[1], R[0]);
    if (ch + 1 < nchunks) step(ch + 1, R[2], R[1]);
    if (ch + 2 < nchunks) step(ch + 2, R[3], R[2]);
    if (ch + 3 < nchunks) step(ch + 3, R[0], R[3]);
  }

  // ---- logits to LDS: [64 tokens][Ep] fp32 (reuses both buffers) ----------------
  float* L = reinterpret_cast<float*>(&buf[0]);
  const int ldl = Ep + 1;   // padded row: the 32 lanes of a store hit distinct banks
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int et = eh + 2 * i;
    if (32 * et < Ep) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) L[(32 * th + li) * ldl + 32 * et + 8 * q + 4 * lg + j] = acc[i][4 * q + j];
    }
  }
  __syncthreads();

  // ---- per token: softmax, top-k, weights --------------------------------------
  // A quad of 4 lanes per token (the 256 threads cover the 64 tokens): lane q
  // holds the logits of experts 4 i + q in registers, reductions across the
  // quad use DPP quad permutes.  A taken (or absent) expert is NaN.
  {
    constexpr int NPER = 16 * NT;          // experts per lane (E <= 64 NT)
    const int t = tid >> 2, q = tid & 3;
    const bool live = t0 + t < T;
    float* lt = L + t * ldl;
    float v[NPER];
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = 4 * i + q;
      v[i] = e < E ? lt[e] + (bias ? bias[e] : 0.0f) : NAN;
      lm = fmaxf(lm, v[i]);               // fmaxf ignores the NaN
    }
    const float m = quad_max(lm);
    float ls = 0.0f;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (v[i] == v[i]) ls += expf(v[i] - m);
    const float sum = quad_sum(ls);
    const int64_t o = (t0 + t) * k;
    float wsel = 0.0f;
    for (int j = 0; j < k; ++j) {
      // this lane's best: the largest logit, the lower id on ties (ascending
      // i is ascending id); be = kNone when the lane has nothing left
      float bv = -INFINITY;
      int be = kNone;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (v[i] == v[i] && (be == kNone || v[i] > bv)) {
          bv = v[i];
          be = 4 * i + q;
        }
      quad_argmax(bv, be);
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (4 * i + q == be) v[i] = NAN;
      const float pe = expf(bv - m);
      wsel += pe;
      if (q == 0) lt[j] = pe;             // the row's logits are in registers now
      if (q == 0 && live) topk_ids[o + j] = be;
    }
    const float den = renormalize ? wsel : sum;
    if (live)
      for (int j = q; j < k; j += 4) topk_w[o + j] = lt[j] / den;
  }
}

}  // namespace

int launch_router(const uint16_t* x, const uint16_t* gate, const float* bias, int64_t T, int64_t K, int64_t E,
                  int64_t k, int renormalize, int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return MX_OK;
  const unsigned grid = (unsigned)((T + kBT - 1) / kBT);
  const int tiles = (int)((E + 31) / 32), per_wave = (tiles + 1) / 2;
#define MX_ROUTER_LAUNCH(NT)                                                                                  \
  router_kernel<NT><<<dim3(grid), dim3(kThreads), 0, stream>>>(x, gate, bias, T, K, (int)E, (int)k,          \
                                                               renormalize, ids, w)
  if (per_wave <= 1) MX_ROUTER_LAUNCH(1);
  else if (per_wave == 2) MX_ROUTER_LAUNCH(2);
  else MX_ROUTER_LAUNCH(4);
#undef MX_ROUTER_LAUNCH
  return check_launch("moe_router");
}

}  // namespace mxmoe

extern "C" int moe_router(const void* x_bf16, const void* gate_bf16, const float* bias, int64_t T, int64_t K,
                          int64_t E, int64_t k, int renormalize, int32_t* topk_ids, float* topk_w,
                          void* stream) {
  using namespace mxmoe;
  if (T < 0 || K <= 0 || E <= 0 || k <= 0)
    return fail(MX_ERR_INVALID_ARG, "moe_router: bad sizes T=%lld K=%lld E=%lld k=%lld", (long long)T,
                (long long)K, (long long)E, (long long)k);
  if (k > E) return fail(MX_ERR_INVALID_ARG, "moe_router: k=%lld > E=%lld", (long long)k, (long long)E);
  if (E > kMaxE) return fail(MX_ERR_UNSUPPORTED, "moe_router: E=%lld > %d", (long long)E, kMaxE);
  if (K % kCK != 0) return fail(MX_ERR_UNSUPPORTED, "moe_router: K=%lld is not a multiple of %d", (long long)K, kCK);
  if (T > 0 && (!x_bf16 || !gate_bf16 || !topk_ids || !topk_w))
    return fail(MX_ERR_INVALID_ARG, "moe_router: null pointer");
  if (reinterpret_cast<uintptr_t>(x_bf16) % 16 || reinterpret_cast<uintptr_t>(gate_bf16) % 16)
    return fail(MX_ERR_UNSUPPORTED, "moe_router: x and gate must be 16-byte aligned");
  return launch_router(static_cast<const uint16_t*>(x_bf16), static_cast<const uint16_t*>(gate_bf16), bias, T,
                       K, E, k, renormalize, topk_ids, topk_w, as_stream(stream));
}
