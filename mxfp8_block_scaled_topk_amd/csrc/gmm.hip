// Grouped MXFP8 GEMMs on CDNA4 block-scaled MFMA.
//
//   gmm_mx              y[m] = bf16( A[m] . W_e^T )                  (GEMM2)
//   gmm_swiglu_mxquant  h[m] = silu(A[m].Wg_e^T) * (A[m].Wu_e^T),
//                       then MX quantisation of h along I            (GEMM1)
//
// Product orientation.  The MFMA "A" operand is a tile of weight rows (output
// features n) and the "B" operand a tile of token rows m, so each lane ends
// up holding 4 consecutive output features of one token: GEMM2 stores 8-byte
// bf16 runs and GEMM1's 32-wide MX block of h sits in two lanes (l, l^32).
//
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 operand layout (measured on gfx950): lane l
// holds row l%32; of its 32 bytes, bytes 0-15 belong to scale block 0 and
// bytes 16-31 to block 1 of the 64-wide K step, with lane group g = l/32
// supplying K [16g, 16g+16) of each block; A and B bytes pair by (g, byte).
// The scale of (row r, block b) is the selected byte of lane r + 32*b's scale
// register.  Output: lane l holds column l%32, rows 8q + 4*(l/32) + (0..3) in
// accumulator elements 4q..4q+3.
//
// Tiling.  A workgroup of 4 waves computes a 128 (weight rows) x 128 (tokens)
// tile; each wave a 64 x 64 quarter as 2 x 2 MFMA tiles.  K advances 128
// bytes per step through an LDS double buffer (16 KB per operand per stage,
// rows of 128 bytes with the 16-byte chunk index XOR-ed by row%8 so the 32
// lanes reading one chunk column hit distinct banks).  Scales for the step
// (4 bytes per row) are staged next to the tiles.
//
// Scheduling.  The kernel is persistent: every workgroup derives the
// per-expert row ranges and m-tile prefix from the device-resident group
// list (no host synchronisation), then walks tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ...; tile t is m-tile t / n_tiles (an m-tile never
// straddles two experts) and n-tile t % n_tiles.  Skewed and empty experts
// cost nothing beyond their own tiles.
#include <algorithm>

#include "common.h"

namespace mxmoe {

namespace {

constexpr int BM = 128;  // token rows per tile
constexpr int BN = 128;  // weight rows per tile
constexpr int BK = 128;  // K bytes per step
constexpr int kThreads = 256;
constexpr int kMaxE = 1024;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct GmmParams {
  const uint8_t* a;    // [M, Kd] e4m3
  const uint8_t* as;   // [M, Kd/32] e8m0
  const uint8_t* w;    // [E, Nw, Kd] e4m3
  const uint8_t* ws;   // [E, Nw, Kd/32] e8m0
  const int64_t* group_list;
  int gl_type;
  int E;
  int64_t M;
  int64_t Kd;
  int64_t Nw;          // weight rows per expert (2I for GEMM1, N for GEMM2)
  int n_tiles;         // tiles along the output features
  int64_t I;           // GEMM1: intermediate size
  uint16_t* y;         // GEMM2 output [M, Nw] bf16
  uint8_t* hq;         // GEMM1 outputs
  uint8_t* hs;
  float* hdbg;
};

__device__ __forceinline__ int64_t group_count(const int64_t* gl, int type, int e) {
  if (type == 1) return gl[e];
  return gl[e] - (e > 0 ? gl[e - 1] : 0);
}

template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void gmm_kernel(GmmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BN * BK];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BM * BK];
  __shared__ uint32_t sSA[2][BN];
  __shared__ uint32_t sSB[2][BM];
  __shared__ int s_tile0[kMaxE + 1];
  __shared__ int s_row0[kMaxE];
  __shared__ int s_row1[kMaxE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E;

  // ---- per-expert row ranges and m-tile prefix (wave 0) -------------------
  if (wave == 0) {
    constexpr int PER = kMaxE / 64;
    int64_t n[PER];
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      int64_t v = e < E ? group_count(p.group_list, p.gl_type, e) : 0;
      v = v < 0 ? 0 : (v > p.M ? p.M : v);
      n[i] = v;
      local += v;
    }
    int64_t x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    int64_t run = x - local;
    int tiles[PER];
    int tloc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      const int64_t r0 = run < p.M ? run : p.M;
      const int64_t r1 = run + n[i] < p.M ? run + n[i] : p.M;
      tiles[i] = (int)((r1 - r0 + BM - 1) / BM);
      if (e < E) {
        s_row0[e] = (int)r0;
        s_row1[e] = (int)r1;
      }
      tloc += tiles[i];
      run += n[i];
    }
    int tx = tloc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(tx, off);
      if (lane >= off) tx += y;
    }
    int trun = tx - tloc;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      if (e < E) s_tile0[e] = trun;
      trun += tiles[i];
    }
    if (lane == 63) s_tile0[E] = tx;
  }
  __syncthreads();

  const int n_tiles = p.n_tiles;
  const int total = s_tile0[E] * n_tiles;
  const int64_t Kd = p.Kd;
  const int64_t srow = Kd / 32;  // scale bytes per row
  const int nk = (int)(Kd / BK);
  const int wn = wave & 1, wm = wave >> 1;
  const int li = lane & 31, lg = lane >> 5;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mt = tile / n_tiles, nt = tile - mt * n_tiles;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tile0[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int64_t m0 = s_row0[e] + (int64_t)(mt - s_tile0[e]) * BM;
    const int64_t m_end = s_row1[e];
    const int rows_valid = (int)std::min<int64_t>(BM, m_end - m0);

    const uint8_t* we = p.w + (int64_t)e * p.Nw * Kd;
    const uint8_t* wse = p.ws + (int64_t)e * p.Nw * srow;

    // weight row (within the expert) held in tile row r
    auto wrow = [&](int r) -> int64_t {
      if (kSwiglu) {
        const int64_t hc0 = (int64_t)nt * 64;
        const int half = r >> 6, q = r & 63;
        return q < 32 ? hc0 + 32 * half + q : p.I + hc0 + 32 * half + (q - 32);
      }
      return (int64_t)nt * BN + r;
    };
    auto arow = [&](int r) -> int64_t { return std::min<int64_t>(m0 + r, m_end - 1); };

    // per-thread global sources and LDS destinations of the 4+4 chunks
    const uint8_t* gA[4];
    const uint8_t* gB[4];
    int lds_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + kThreads * i;
      const int r = q >> 3, c = q & 7;
      gA[i] = we + wrow(r) * Kd + c * 16;
      gB[i] = p.a + arow(r) * Kd + c * 16;
      lds_off[i] = r * BK + ((c ^ (r & 7)) << 4);
    }
    const uint8_t* gS = tid < BN ? wse + wrow(tid) * srow : p.as + arow(tid - BN) * srow;

    // Register-staged double buffer: step ks computes from LDS buffer ks&1
    // while the loads of step ks+1 are in flight; the last step re-loads
    // step nk-1 (in bounds, result unused) so the loop has no branches.
    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
    uint32_t rs;
#define MX_GMM_LOAD(ks_)                                                  \
    do {                                                                  \
      const int64_t o_ = (int64_t)(ks_) * BK;                             \
      ra0 = *reinterpret_cast<const uint4*>(gA[0] + o_);                  \
      ra1 = *reinterpret_cast<const uint4*>(gA[1] + o_);                  \
      ra2 = *reinterpret_cast<const uint4*>(gA[2] + o_);                  \
      ra3 = *reinterpret_cast<const uint4*>(gA[3] + o_);                  \
      rb0 = *reinterpret_cast<const uint4*>(gB[0] + o_);                  \
      rb1 = *reinterpret_cast<const uint4*>(gB[1] + o_);                  \
      rb2 = *reinterpret_cast<const uint4*>(gB[2] + o_);                  \
      rb3 = *reinterpret_cast<const uint4*>(gB[3] + o_);                  \
      rs = *reinterpret_cast<const uint32_t*>(gS + (int64_t)(ks_) * 4);   \
    } while (0)
#define MX_GMM_STORE(buf_)                                                \
    do {                                                                  \
      *reinterpret_cast<uint4*>(&sA[buf_][lds_off[0]]) = ra0;             \
      *reinterpret_cast<uint4*>(&sA[buf_][lds_off[1]]) = ra1;             \
      *reinterpret_cast<uint4*>(&sA[buf_][lds_off[2]]) = ra2;             \
      *reinterpret_cast<uint4*>(&sA[buf_][lds_off[3]]) = ra3;             \
      *reinterpret_cast<uint4*>(&sB[buf_][lds_off[0]]) = rb0;             \
      *reinterpret_cast<uint4*>(&sB[buf_][lds_off[1]]) = rb1;             \
      *reinterpret_cast<uint4*>(&sB[buf_][lds_off[2]]) = rb2;             \
      *reinterpret_cast<uint4*>(&sB[buf_][lds_off[3]]) = rb3;             \
      if (tid < BN) sSA[buf_][tid] = rs; else sSB[buf_][tid - BN] = rs;   \
    } while (0)

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    MX_GMM_LOAD(0);
    MX_GMM_STORE(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      MX_GMM_LOAD(ks + 1 < nk ? ks + 1 : ks);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c0 = 4 * s + lg, c1 = 4 * s + 2 + lg;
        v8i fa[2], fb[2];
        int sa[2], sb[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int ra_ = 64 * wn + 32 * f + li;
          const uint8_t* baseA = &sA[buf][ra_ * BK];
          const uint4 a0 = *reinterpret_cast<const uint4*>(baseA + ((c0 ^ (ra_ & 7)) << 4));
          const uint4 a1 = *reinterpret_cast<const uint4*>(baseA + ((c1 ^ (ra_ & 7)) << 4));
          fa[f] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          sa[f] = (int)(sSA[buf][ra_] >> (8 * (2 * s + lg)));
          const int rb_ = 64 * wm + 32 * f + li;
          const uint8_t* baseB = &sB[buf][rb_ * BK];
          const uint4 b0 = *reinterpret_cast<const uint4*>(baseB + ((c0 ^ (rb_ & 7)) << 4));
          const uint4 b1 = *reinterpret_cast<const uint4*>(baseB + ((c1 ^ (rb_ & 7)) << 4));
          fb[f] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          sb[f] = (int)(sSB[buf][rb_] >> (8 * (2 * s + lg)));
        }
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int fm = 0; fm < 2; ++fm)
            acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[fn], fb[fm], acc[fn][fm], 0, 0, 0, sa[fn], 0, sb[fm]);
      }
      MX_GMM_STORE(buf ^ 1);
      __syncthreads();
    }
#undef MX_GMM_LOAD
#undef MX_GMM_STORE

    // ---- epilogue ----------------------------------------------------------
    if (!kSwiglu) {
      const int64_t N = p.Nw;
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) {
        const int mc = 64 * wm + 32 * fm + li;
        if (mc >= rows_valid) continue;
        uint16_t* yrow = p.y + (m0 + mc) * N + (int64_t)nt * BN + 64 * wn;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v16f& c = acc[fn][fm];
            uint2 o;
            o.x = f32_to_bf16(c[4 * q]) | (f32_to_bf16(c[4 * q + 1]) << 16);
            o.y = f32_to_bf16(c[4 * q + 2]) | (f32_to_bf16(c[4 * q + 3]) << 16);
            *reinterpret_cast<uint2*>(yrow + 32 * fn + 8 * q + 4 * lg) = o;
          }
      }
    } else {
      const int64_t I = p.I;
      const int64_t hcol0 = (int64_t)nt * 64 + 32 * wn;   // first h column of this wave's block
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) {
        const int mc = 64 * wm + 32 * fm + li;
        const bool ok = mc < rows_valid;
        float h[16];
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float g = acc[0][fm][v], u = acc[1][fm][v];
          h[v] = g / (1.0f + __expf(-g)) * u;
          amax = fmaxf(amax, fabsf(h[v]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const uint32_t sbyte = e8m0_from_amax(amax);
        const float inv = e8m0_inverse(sbyte);
        if (ok) {
          const int64_t m = m0 + mc;
          uint8_t* hrow = p.hq + m * I + hcol0;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint32_t*>(hrow + 8 * q + 4 * lg) =
                e4m3x4(h[4 * q] * inv, h[4 * q + 1] * inv, h[4 * q + 2] * inv, h[4 * q + 3] * inv);
          if (lg == 0) p.hs[m * (I / 32) + hcol0 / 32] = static_cast<uint8_t>(sbyte);
          if (p.hdbg) {
            float* drow = p.hdbg + m * I + hcol0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(drow + 8 * q + 4 * lg) =
                  make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
          }
        }
      }
    }
  }
}

int g_occ[2] = {0, 0};

template <bool kSwiglu>
int launch(const GmmParams& p, hipStream_t stream, const char* name) {
  if (p.M == 0) return MX_OK;
  int& occ = g_occ[kSwiglu ? 1 : 0];
  if (occ == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gmm_kernel<kSwiglu>, kThreads, 0) != hipSuccess || n <= 0)
      n = 1;
    occ = n;
  }
  const int64_t upper = ((p.M + BM - 1) / BM + p.E) * (int64_t)p.n_tiles;
  const int64_t grid = std::min<int64_t>(upper, (int64_t)num_cus() * occ);
  gmm_kernel<kSwiglu><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(p);
  return check_launch(name);
}

}  // namespace

int check_gmm_common(const char* name, int gl_type, int64_t M, int64_t Kd, int64_t E) {
  if (M < 0 || Kd <= 0 || E <= 0)
    return fail(MX_ERR_INVALID_ARG, "%s: bad sizes M=%lld K=%lld E=%lld", name, (long long)M, (long long)Kd,
                (long long)E);
  if (gl_type != 0 && gl_type != 1)
    return fail(MX_ERR_INVALID_ARG, "%s: group_list_type must be 0 (cumulative) or 1 (count), got %d", name,
                gl_type);
  if (Kd % BK != 0) return fail(MX_ERR_UNSUPPORTED, "%s: reduction size %lld is not a multiple of %d", name,
                                (long long)Kd, BK);
  if (E > kMaxE) return fail(MX_ERR_UNSUPPORTED, "%s: E=%lld > %d", name, (long long)E, kMaxE);
  if (M >= (int64_t)1 << 31) return fail(MX_ERR_UNSUPPORTED, "%s: M >= 2^31", name);
  return MX_OK;
}

int launch_gmm_mx(const uint8_t* a, const uint8_t* as, const uint8_t* w, const uint8_t* ws,
                  const int64_t* gl, int gl_type, int64_t M, int64_t N, int64_t Kd, int64_t E, uint16_t* y,
                  hipStream_t stream) {
  GmmParams p{};
  p.a = a; p.as = as; p.w = w; p.ws = ws; p.group_list = gl; p.gl_type = gl_type;
  p.E = (int)E; p.M = M; p.Kd = Kd; p.Nw = N; p.n_tiles = (int)(N / BN); p.y = y;
  return launch<false>(p, stream, "gmm_mx");
}

int launch_gmm_swiglu(const uint8_t* a, const uint8_t* as, const uint8_t* w13, const uint8_t* w13s,
                      const int64_t* gl, int gl_type, int64_t M, int64_t K, int64_t I, int64_t E, uint8_t* hq,
                      uint8_t* hs, float* hdbg, hipStream_t stream) {
  GmmParams p{};
  p.a = a; p.as = as; p.w = w13; p.ws = w13s; p.group_list = gl; p.gl_type = gl_type;
  p.E = (int)E; p.M = M; p.Kd = K; p.Nw = 2 * I; p.n_tiles = (int)(I / 64); p.I = I;
  p.hq = hq; p.hs = hs; p.hdbg = hdbg;
  return launch<true>(p, stream, "gmm_swiglu_mxquant");
}

}  // namespace mxmoe

extern "C" int gmm_mx(const void* a_u8, const void* a_s, const void* w_u8, const void* w_s,
                      const int64_t* group_list, int group_list_type, int64_t M, int64_t N, int64_t Kd,
                      int64_t E, void* y_bf16, void* stream) {
  using namespace mxmoe;
  int rc = check_gmm_common("gmm_mx", group_list_type, M, Kd, E);
  if (rc) return rc;
  if (N <= 0) return fail(MX_ERR_INVALID_ARG, "gmm_mx: bad N=%lld", (long long)N);
  if (N % BN != 0) return fail(MX_ERR_UNSUPPORTED, "gmm_mx: N=%lld is not a multiple of %d", (long long)N, BN);
  if (!group_list || (M > 0 && (!a_u8 || !a_s || !w_u8 || !w_s || !y_bf16)))
    return fail(MX_ERR_INVALID_ARG, "gmm_mx: null pointer");
  if (reinterpret_cast<uintptr_t>(a_u8) % 16 || reinterpret_cast<uintptr_t>(w_u8) % 16 ||
      reinterpret_cast<uintptr_t>(a_s) % 4 || reinterpret_cast<uintptr_t>(w_s) % 4 ||
      reinterpret_cast<uintptr_t>(y_bf16) % 8)
    return fail(MX_ERR_UNSUPPORTED, "gmm_mx: misaligned pointer");
  return launch_gmm_mx(static_cast<const uint8_t*>(a_u8), static_cast<const uint8_t*>(a_s),
                       static_cast<const uint8_t*>(w_u8), static_cast<const uint8_t*>(w_s), group_list,
                       group_list_type, M, N, Kd, E, static_cast<uint16_t*>(y_bf16), as_stream(stream));
}

extern "C" int gmm_swiglu_mxquant(const void* a_u8, const void* a_s, const void* w13_u8, const void* w13_s,
                                  const int64_t* group_list, int group_list_type, int64_t M, int64_t K,
                                  int64_t I, int64_t E, void* hq_u8, void* hs_u8, float* h_f32_debug,
                                  void* stream) {
  using namespace mxmoe;
  int rc = check_gmm_common("gmm_swiglu_mxquant", group_list_type, M, K, E);
  if (rc) return rc;
  if (I <= 0) return fail(MX_ERR_INVALID_ARG, "gmm_swiglu_mxquant: bad I=%lld", (long long)I);
  if (I % 64 != 0)
    return fail(MX_ERR_UNSUPPORTED, "gmm_swiglu_mxquant: I=%lld is not a multiple of 64", (long long)I);
  if (!group_list || (M > 0 && (!a_u8 || !a_s || !w13_u8 || !w13_s || !hq_u8 || !hs_u8)))
    return fail(MX_ERR_INVALID_ARG, "gmm_swiglu_mxquant: null pointer");
  if (reinterpret_cast<uintptr_t>(a_u8) % 16 || reinterpret_cast<uintptr_t>(w13_u8) % 16 ||
      reinterpret_cast<uintptr_t>(a_s) % 4 || reinterpret_cast<uintptr_t>(w13_s) % 4 ||
      reinterpret_cast<uintptr_t>(hq_u8) % 4 || reinterpret_cast<uintptr_t>(h_f32_debug) % 16)
    return fail(MX_ERR_UNSUPPORTED, "gmm_swiglu_mxquant: misaligned pointer");
  return launch_gmm_swiglu(static_cast<const uint8_t*>(a_u8), static_cast<const uint8_t*>(a_s),
                           static_cast<const uint8_t*>(w13_u8), static_cast<const uint8_t*>(w13_s), group_list,
                           group_list_type, M, K, I, E, static_cast<uint8_t*>(hq_u8),
                           static_cast<uint8_t*>(hs_u8), h_f32_debug, as_stream(stream));
}
