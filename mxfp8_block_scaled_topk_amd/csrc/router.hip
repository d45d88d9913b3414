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
// One workgroup of 8 waves (two per SIMD) handles 64 tokens.  The gate GEMM
// runs on the bf16 MFMA (V_MFMA_F32_32X32X16_BF16: lane l holds operand row
// l % 32 and the 8 k-values [8 (l/32), 8 (l/32) + 8) of the 16-wide step;
// output lane l holds column l % 32 and rows 8 q + 4 (l/32) + (0..3) in
// accumulator elements 4 q .. 4 q + 3).  Gate rows are the A operand
// (experts), token rows the B operand.  K advances 64 values (128 bytes per
// row) per chunk through a ring of S LDS slots, each holding the 64 token rows
// and the gate rows of one chunk, filled by direct global->LDS loads (1 KB =
// 8 rows per instruction, no staging registers) running S-1 chunks ahead
// (measured: a 4-deep ring of register sets, about 72 KB in flight per CU,
// ran 0.78 us per chunk).  16-byte chunk c of row r sits at chunk c ^ (r % 8),
// which keeps the fragment reads (32 rows, one chunk) spread over the LDS
// banks; the swizzle is applied on the global side by choosing which chunk
// each DMA lane fetches.  Wave w covers tokens 32 (w % 2) .. + 32 and expert
// tiles w / 2, w / 2 + 4, ...  The logits then go through LDS to 8 lanes per
// token for the softmax and the selection (measured: one thread per token
// walking its row in LDS took two thirds of the kernel's time; with one wave
// per SIMD the selection's dependency chains were latency-bound).  HBM-bound:
// x is read once (2 T K bytes), the gate comes from L2.
#include "common.h"

namespace mxmoe {

namespace {

constexpr int kThreads = 512;   // 8 waves, two per SIMD
constexpr int kBT = 64;        // tokens per workgroup
constexpr int kCK = 64;        // k values per chunk (128 bytes of a row)
constexpr int kMaxE = 256;
constexpr int kRow = kCK * 2;  // bytes per row per chunk

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// LDS ring: slots of 64 token rows then Ep gate rows, 128 bytes each; Ep <=
// 64 NT rows.  Slots per ring: as many as fit in 160 KB, at most 6.
template <int NT>
struct Ring {
  static constexpr int kSlotBytes = (kBT + 64 * NT) * kRow;
  static constexpr int kSlots = (160 * 1024) / kSlotBytes < 6 ? (160 * 1024) / kSlotBytes : 6;
};

// 64 lanes x 16 B from global (uniform base + per-lane 32-bit offset) to LDS
// [m0, m0 + 1024).
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

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
// The other quad of the lane's aligned group of 8 (DPP row_half_mirror: lane
// i of each 8 takes lane 7 - i).  Applied to a value that is uniform within
// each quad, it swaps the group's two quads, with no trip through the LDS
// unit as a ds_swizzle exchange would take.
constexpr int kHalfMirror = 0x141;
__device__ __forceinline__ int other_quad(int x) {
  return __builtin_amdgcn_update_dpp(x, x, kHalfMirror, 0xf, 0xf, false);
}
__device__ __forceinline__ float other_quadf(float x) { return __int_as_float(other_quad(__float_as_int(x))); }
// Reductions over the 8 lanes (an aligned group) that hold one token: within
// each quad, then across the group's two quads.
__device__ __forceinline__ float oct_max(float x) {
  x = fmaxf(x, quad_swapf1(x));
  x = fmaxf(x, quad_swapf2(x));
  return fmaxf(x, other_quadf(x));
}
__device__ __forceinline__ float oct_sum(float x) {
  x += quad_swapf1(x);
  x += quad_swapf2(x);
  return x + other_quadf(x);
}
__device__ __forceinline__ int oct_min(int x) {
  x = min(x, quad_swap<kQuadXor1>(x));
  x = min(x, quad_swap<kQuadXor2>(x));
  return min(x, other_quad(x));
}
template <int NT>   // gate rows held per chunk: 64 NT (E <= 64 NT)
__global__ __launch_bounds__(kThreads) void router_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gate,
                                                          const float* __restrict__ bias, int64_t T, int64_t K,
                                                          int E, int k, int renormalize,
                                                          int32_t* __restrict__ topk_ids,
                                                          float* __restrict__ topk_w) {
  constexpr int kS = Ring<NT>::kSlots;
  constexpr int kSlotBytes = Ring<NT>::kSlotBytes;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kS * kSlotBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * kBT;
  const int Ep = (E + 31) & ~31;   // expert rows held in LDS
  const int nchunks = (int)(K / kCK);

  // ---- the DMA of one chunk --------------------------------------------------------
  // Instruction i fills LDS rows [8 i, 8 i + 8) of the slot: i < 8 token rows,
  // then 8 NT instructions of gate rows (64 NT rows, the tier's maximum, so
  // every wave issues the same kOps per chunk whatever E is); wave w issues
  // i = w, w + 8, ...  Lane l lands at row 8 i + l/8, physical chunk l%8, and
  // fetches logical chunk (l%8) ^ ((l/8)%8).  Rows past T or E repeat the last
  // row (their logits are never selected or stored).
  constexpr int kOps = (8 + 8 * NT) / 8;   // per wave per chunk
  const int lrow = lane >> 3, lchk = (lane & 7) ^ (lrow & 7);
  const uint32_t ring_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)ring;
  const int tlast = (int)(T - 1 - t0 < kBT - 1 ? T - 1 - t0 : kBT - 1);   // last readable token row
  const uint16_t* xrow = x + t0 * K;
  auto dma_chunk = [&](int ch, int slot) __attribute__((always_inline)) {
    const uint32_t sbase = ring_base + (uint32_t)(slot * kSlotBytes);
#pragma unroll
    for (int j = 0; j < kOps; ++j) {
      const int i = wave + 8 * j;
      int r = 8 * i + lrow;   // LDS row in the slot
      const void* base;
      uint32_t voff;
      if (i < 8) {
        const int tr = r < tlast ? r : tlast;
        base = xrow;
        voff = (uint32_t)(tr * K * 2 + ch * kRow + lchk * 16);
      } else {
        const int er = r - kBT < E - 1 ? r - kBT : E - 1;
        base = gate;
        voff = (uint32_t)(er * K * 2 + ch * kRow + lchk * 16);
      }
      dma16(voff, base, sbase + (uint32_t)(8 * i * kRow));
    }
  };

  // wave w: tokens 32 (w % 2) .. + 32, expert tiles w/2, w/2 + 4, ...
  constexpr int NTW = NT > 1 ? NT / 2 : 1;   // expert tiles per wave
  const int th = wave & 1, eh = wave >> 1;
  const int li = lane & 31, lg = lane >> 5;
  v16f acc[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  // All of a chunk's fragment reads go out before its MFMAs, so their LDS
  // latencies overlap (one wave per SIMD: nothing else hides them).
  auto mfma_chunk = [&](int slot) __attribute__((always_inline)) {
    const uint8_t* bx = ring + slot * kSlotBytes;
    const uint8_t* bg = bx + kBT * kRow;
    bf16x8 xb[kCK / 16], gb[kCK / 16][NTW];
#pragma unroll
    for (int s = 0; s < kCK / 16; ++s) {
      const int c = 2 * s + lg;   // this lane's 16-byte chunk of the step
      xb[s] = *reinterpret_cast<const bf16x8*>(bx + swz(32 * th + li, c));
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int et = eh + 4 * i;
        const int er = 32 * et < Ep ? 32 * et + li : li;   // absent tiles read a valid row, unused
        gb[s][i] = *reinterpret_cast<const bf16x8*>(bg + swz(er, c));
      }
    }
#pragma unroll
    for (int s = 0; s < kCK / 16; ++s)
#pragma unroll
      for (int i = 0; i < NTW; ++i)
        if (32 * (eh + 4 * i) < Ep) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gb[s][i], xb[s], acc[i], 0, 0, 0);
  };

  // prologue: chunks 0 .. kS-2 in flight; chunk ch lives in slot ch % kS
  for (int c = 0; c < kS - 1; ++c)
    if (c < nchunks) dma_chunk(c, c);
  for (int ch = 0; ch < nchunks; ++ch) {
    // this wave's part of chunk ch has landed once at most the kS-2 later
    // chunks' loads are outstanding (loads retire in order; near the end,
    // with fewer later chunks issued, wait for all); the barrier makes every
    // wave's part visible and frees the slot of chunk ch - 1
    if (ch + kS - 2 < nchunks)
      wait_vmcnt<(kS - 2) * kOps>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    // the MFMAs first: a DMA issue can stall the wave while the memory
    // pipeline is full, and the matrix work should not wait behind it
    mfma_chunk(ch % kS);
    if (ch + kS - 1 < nchunks) dma_chunk(ch + kS - 1, (ch + kS - 1) % kS);
  }
  __syncthreads();

  // ---- logits to LDS: [64 tokens][Ep] fp32 (reuses the ring) ---------------------
  float* L = reinterpret_cast<float*>(ring);
  const int ldl = Ep + 1;   // padded row: the 32 lanes of a store hit distinct banks
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int et = eh + 4 * i;
    if (32 * et < Ep) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) L[(32 * th + li) * ldl + 32 * et + 8 * q + 4 * lg + j] = acc[i][4 * q + j];
    }
  }
  __syncthreads();

  // ---- per token: softmax, top-k, weights --------------------------------------
  // 8 lanes per token (the 512 threads cover the 64 tokens): lane q holds the
  // logits of experts 8 i + q in registers; reductions across the 8 use DPP
  // permutes only.  A taken (or absent) expert is NaN.
  {
    constexpr int NPER = 8 * NT;           // experts per lane (E <= 64 NT)
    const int t = tid >> 3, q = tid & 7;
    const bool live = t0 + t < T;
    float* lt = L + t * ldl;
    float v[NPER];
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = 8 * i + q;
      v[i] = e < E ? lt[e] + (bias ? bias[e] : 0.0f) : NAN;
      lm = fmaxf(lm, v[i]);               // fmaxf ignores the NaN
    }
    const float m = oct_max(lm);
    // four partial sums: independent chains
    float ls4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (v[i] == v[i]) ls4[i & 3] += __expf(v[i] - m);
    const float sum = oct_sum((ls4[0] + ls4[1]) + (ls4[2] + ls4[3]));
    const int64_t o = (t0 + t) * k;
    float wsel = 0.0f;
    for (int j = 0; j < k; ++j) {
      // the token's best: the largest remaining logit (a max tree over the
      // lane's values, fmaxf ignoring the NaN of taken experts, then over the
      // token's 8 lanes), and among equal ones the lowest id (a min tree over the ids
      // holding that value); trees instead of one running comparison keep the
      // dependency chains short
      float t[NPER];
#pragma unroll
      for (int i = 0; i < NPER; ++i) t[i] = v[i];
#pragma unroll
      for (int w = NPER / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
      const float bv = oct_max(t[0]);
      int c[NPER];
#pragma unroll
      for (int i = 0; i < NPER; ++i) c[i] = v[i] == bv ? 8 * i + q : kNone;
#pragma unroll
      for (int w = NPER / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) c[i] = c[i] < c[i + w] ? c[i] : c[i + w];
      const int be = oct_min(c[0]);
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (8 * i + q == be) v[i] = NAN;
      const float pe = __expf(bv - m);
      wsel += pe;
      if (q == 0) lt[j] = pe;             // the row's logits are in registers now
      if (q == 0 && live) topk_ids[o + j] = be;
    }
    const float den = renormalize ? wsel : sum;
    if (live)
      for (int j = q; j < k; j += 8) topk_w[o + j] = lt[j] / den;
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
  if (!dims_in_range({T, K})) return fail(MX_ERR_UNSUPPORTED, "moe_router: T or K above 2^31 - 1");
  if (E > kMaxE) return fail(MX_ERR_UNSUPPORTED, "moe_router: E=%lld > %d", (long long)E, kMaxE);
  if (K % kCK != 0) return fail(MX_ERR_UNSUPPORTED, "moe_router: K=%lld is not a multiple of %d", (long long)K, kCK);
  if (T > 0 && (!x_bf16 || !gate_bf16 || !topk_ids || !topk_w))
    return fail(MX_ERR_INVALID_ARG, "moe_router: null pointer");
  if (reinterpret_cast<uintptr_t>(x_bf16) % 16 || reinterpret_cast<uintptr_t>(gate_bf16) % 16)
    return fail(MX_ERR_UNSUPPORTED, "moe_router: x and gate must be 16-byte aligned");
  return launch_router(static_cast<const uint16_t*>(x_bf16), static_cast<const uint16_t*>(gate_bf16), bias, T,
                       K, E, k, renormalize, topk_ids, topk_w, as_stream(stream));
}
