// moe_route_quant: top-k routing with the MX activation quant fused in.
//
// The T*k assignments (flat index i = t*k + j) are cut into chunks of whole
// tokens, at most 256 assignments each (one per thread).  Three launches:
//
//   route_hist           per chunk, per expert assignment counts (LDS atomics;
//                        counts are order-free so atomics keep it exact)
//   route_scan           one wave per expert: exclusive prefix of its counts
//                        over the chunks, plus the expert's total (= group_list)
//   route_scatter_quant  kSplit blocks per chunk: each finds the stable rank of
//                        every assignment among the chunk's assignments to
//                        the same expert (wave ballot match + per-wave counts
//                        in LDS), hence its row p = offset[e] +
//                        prefix[e][chunk] + rank; the first block writes both
//                        maps; then each block MX-quantises its share of the
//                        chunk's tokens once, in registers (two lanes per
//                        32-element block, the block's amax combined with
//                        one lane exchange), and stores the payload and
//                        scales to each token's k rows: every store
//                        instruction writes 1 KB of one row contiguously.
//                        Several blocks per chunk keep enough waves resident
//                        to hide the load latency (one block per chunk left
//                        the kernel at about 8 waves per CU at the 16K
//                        prefill size).  Most of its traffic is HBM writes
//                        (k quantised copies of every token).
//
// When all T*k assignments fit in one chunk (decode-sized batches) the
// histogram and scan launches are skipped: the scatter blocks take the
// experts' totals from their own per-wave counts (prefix 0 for the only
// chunk), and the first block writes the group list.
//
// The order inside an expert is the flat index order, so the permutation is
// deterministic and equals a stable sort by expert.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace mxmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 1024;
// blocks per routing chunk in route_scatter_quant (each ranks the whole
// chunk, then quantises its share of the tokens); measured in the layer's
// kernel sequence at the 16K prefill size: 4: 89.6 us (in a loop of routing
// calls), 8: 71.7 us, 16: 68.7 us, 32: 98.8 us
constexpr int kSplit = 16;

__global__ __launch_bounds__(kThreads) void route_hist(const int32_t* __restrict__ ids, int64_t M,
                                                       int k, int E, int tpc, int nchunks,
                                                       int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int c = blockIdx.x;
  const int64_t a = (int64_t)c * tpc * k + threadIdx.x;
  if ((int)threadIdx.x < tpc * k && a < M) {
    const int e = ids[a];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) counts[(int64_t)e * nchunks + c] = hist[e];
}

// counts [E][nchunks] -> exclusive prefix over chunks (in place); totals[e].
__global__ __launch_bounds__(kThreads) void route_scan(int32_t* __restrict__ counts, int nchunks, int E,
                                                       int32_t* __restrict__ totals,
                                                       int64_t* __restrict__ group_list) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kThreads / 64) + wave;
  if (e >= E) return;  // uniform per wave
  int32_t* row = counts + (int64_t)e * nchunks;
  int run = 0;
  // 512 chunks per round, 8 consecutive ones per lane: all loads of a round
  // are in flight together (one memory round trip per 512 chunks)
  for (int base = 0; base < nchunks; base += 512) {
    const int i0 = base + 8 * lane;
    int v[8];
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = i0 + j < nchunks ? row[i0 + j] : 0;
      s += v[j];
    }
    const int x = wave_inclusive_scan(s);
    int excl = run + x - s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (i0 + j < nchunks) row[i0 + j] = excl;
      excl += v[j];
    }
    run += __builtin_amdgcn_readlane(x, 63);
  }
  if (lane == 0) {
    totals[e] = run;
    group_list[e] = run;
  }
}

// Exclusive scan of v[0..n) (n <= 1024) into out[0..n) by one 256-thread block.
// Every read of v precedes the block barrier inside and every write to out
// follows it, so out may be v (in place).
__device__ void block_exclusive_scan(const int32_t* v, int n, int* out, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int loc[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    loc[i] = e < n ? v[e] : 0;
    sum += loc[i];
  }
  const int x = wave_inclusive_scan(sum);
  if (lane == 63) s_wsum[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  int run = base + x - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < n) out[e] = run;
    run += loc[i];
  }
}

__global__ __launch_bounds__(kThreads) void route_scatter_quant(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, int64_t T, int64_t K, int k,
    int E, int nbits, int tpc, int nchunks, const int32_t* __restrict__ prefix,
    const int32_t* __restrict__ totals, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
    int32_t* __restrict__ sorted_row, int32_t* __restrict__ eri, int64_t* __restrict__ group_list) {
  __shared__ int s_off[kMaxE];
  __shared__ int s_wcnt[kThreads / 64][kMaxE];
  __shared__ int s_pos[kThreads];
  __shared__ int s_wsum[kThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x / kSplit, part = blockIdx.x % kSplit;
  for (int w = 0; w < kThreads / 64; ++w)
    for (int e = tid; e < E; e += kThreads) s_wcnt[w][e] = 0;
  const bool single = nchunks == 1;   // no histogram / scan launches (see the header)
  if (!single) block_exclusive_scan(totals, E, s_off, s_wsum);
  __syncthreads();

  // ---- stable rank of each assignment within the chunk -------------------
  const int64_t M = T * k;
  const int64_t a0 = (int64_t)c * tpc * k;
  const int na = (int)std::min<int64_t>((int64_t)tpc * k, M - a0);
  const int64_t a = a0 + tid;
  int e = 0;
  bool valid = false;
  if (tid < na) {
    e = ids[a];
    valid = e >= 0 && e < E;
  }
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t ones = __ballot(bit);
    same &= bit ? ones : ~ones;
  }
  int rank = __popcll(same & ((1ull << lane) - 1ull));
  if (valid && rank == 0) s_wcnt[wave][e] = __popcll(same);
  __syncthreads();
  if (single) {
    // the only chunk's counts are the experts' totals
    for (int ee = tid; ee < E; ee += kThreads) {
      int n = 0;
      for (int w = 0; w < kThreads / 64; ++w) n += s_wcnt[w][ee];
      s_off[ee] = n;
      if (part == 0) group_list[ee] = n;
    }
    __syncthreads();
    block_exclusive_scan(s_off, E, s_off, s_wsum);
    __syncthreads();
  }
  int pos = -1;
  if (valid) {
    for (int w = 0; w < wave; ++w) rank += s_wcnt[w][e];
    pos = s_off[e] + (single ? 0 : prefix[(int64_t)e * nchunks + c]) + rank;
    if (part == 0) sorted_row[pos] = (int32_t)a;
  }
  if (part == 0 && tid < na) eri[a] = pos;
  s_pos[tid] = pos;
  __syncthreads();

  // ---- MX quant of the chunk's tokens, stored to each token's k rows ------
  const int64_t nb = K / 32;
  const int64_t s_stride = ((nb + 1) / 2) * 2;
  // this block's tokens: [tb, te) of the chunk
  const int64_t t0 = (int64_t)c * tpc;
  const int ntok = (int)std::min<int64_t>((int64_t)tpc, T - t0);
  const int per = (tpc + kSplit - 1) / kSplit;
  const int tb = std::min(part * per, ntok), te = std::min(tb + per, ntok);
  const int64_t hpr = 2 * nb;   // half-blocks per token row
  const int64_t items = (int64_t)(te - tb) * hpr;   // even, so lane pairs (2m, 2m+1) stay together
  for (int64_t it = tid; it < items; it += kThreads) {
    const int tl = tb + (int)(it / hpr);
    const int64_t hb = it - (int64_t)(tl - tb) * hpr;
    const int64_t b = hb >> 1;
    const int half = (int)(hb & 1);
    const uint4* src = reinterpret_cast<const uint4*>(x + (t0 + tl) * K + b * 32 + half * 16);
    const uint4 u0 = src[0], u1 = src[1];
    float v[16];
    unpack_bf16x8(u0, v);
    unpack_bf16x8(u1, v + 8);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const uint32_t sb = e8m0_from_amax(amax);
    const float inv = e8m0_inverse(sb);
    uint4 q;
    q.x = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    q.y = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    q.z = e4m3x4(v[8] * inv, v[9] * inv, v[10] * inv, v[11] * inv);
    q.w = e4m3x4(v[12] * inv, v[13] * inv, v[14] * inv, v[15] * inv);
    for (int j = 0; j < k; ++j) {
      const int p = s_pos[tl * k + j];
      if (p < 0) continue;
      *reinterpret_cast<uint4*>(xq + (int64_t)p * K + b * 32 + half * 16) = q;
      if (half == 0) {
        xs[(int64_t)p * s_stride + b] = static_cast<uint8_t>(sb);
        if ((nb & 1) && b == nb - 1) xs[(int64_t)p * s_stride + nb] = 0;
      }
    }
  }
}

__global__ void zero_i64(int64_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

inline int64_t tokens_per_chunk(int64_t k) { return std::max<int64_t>(1, kThreads / k); }
inline int64_t num_chunks(int64_t T, int64_t k) {
  const int64_t tpc = tokens_per_chunk(k);
  return (T + tpc - 1) / tpc;
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int64_t k, int64_t E) {
  const int64_t nch = num_chunks(T, k);
  return align_up((size_t)(E * nch) * 4, 256) + align_up((size_t)E * 4, 256);
}

int check_route_args(int64_t T, int64_t K, int64_t k, int64_t E) {
  if (T < 0 || K <= 0 || k <= 0 || E <= 0)
    return fail(MX_ERR_INVALID_ARG, "moe_route_quant: bad sizes T=%lld K=%lld k=%lld E=%lld",
                (long long)T, (long long)K, (long long)k, (long long)E);
  if (k > E) return fail(MX_ERR_INVALID_ARG, "moe_route_quant: k=%lld > E=%lld", (long long)k, (long long)E);
  if (!dims_in_range({T, K})) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: T or K above 2^31 - 1");
  if (K % 32 != 0) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: K=%lld is not a multiple of 32", (long long)K);
  if (k > kThreads) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: k=%lld > %d", (long long)k, kThreads);
  if (E > kMaxE) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: E=%lld > %d", (long long)E, kMaxE);
  if (T * k >= (int64_t)1 << 31) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: T*k >= 2^31");
  return MX_OK;
}

int launch_route_quant(const uint16_t* x, const int32_t* ids, int64_t T, int64_t K, int64_t k,
                       int64_t E, uint8_t* xq, uint8_t* xs, int32_t* sorted_row, int32_t* eri,
                       int64_t* group_list, void* ws, hipStream_t stream) {
  const int64_t tpc = tokens_per_chunk(k);
  const int64_t nch = num_chunks(T, k);
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* totals = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up((size_t)(E * nch) * 4, 256));
  if (T == 0) {
    zero_i64<<<dim3((unsigned)((E + 255) / 256)), dim3(256), 0, stream>>>(group_list, (int)E);
    return check_launch("moe_route_quant(zero)");
  }
  int nbits = 0;
  while ((1ll << nbits) < E) ++nbits;
  if (nch == 1) {
    route_scatter_quant<<<dim3((unsigned)kSplit), dim3(kThreads), 0, stream>>>(
        x, ids, T, K, (int)k, (int)E, nbits, (int)tpc, 1, nullptr, nullptr, xq, xs, sorted_row, eri, group_list);
    return check_launch("route_scatter_quant");
  }
  route_hist<<<dim3((unsigned)nch), dim3(kThreads), 0, stream>>>(ids, T * k, (int)k, (int)E, (int)tpc,
                                                                   (int)nch, counts);
  int rc = check_launch("route_hist");
  if (rc) return rc;
  route_scan<<<dim3((unsigned)((E + 3) / 4)), dim3(kThreads), 0, stream>>>(counts, (int)nch, (int)E, totals,
                                                                           group_list);
  rc = check_launch("route_scan");
  if (rc) return rc;
  route_scatter_quant<<<dim3((unsigned)(nch * kSplit)), dim3(kThreads), 0, stream>>>(
      x, ids, T, K, (int)k, (int)E, nbits, (int)tpc, (int)nch, counts, totals, xq, xs, sorted_row, eri,
      group_list);
  return check_launch("route_scatter_quant");
}

}  // namespace mxmoe

extern "C" size_t moe_route_quant_workspace_size(int64_t T, int64_t k, int64_t E) {
  // 0 for sizes the routing rejects (the workspace of a call that fails)
  if (mxmoe::check_route_args(T, 32, k, E) != MX_OK) return 0;
  return mxmoe::route_workspace_bytes(T, k, E);
}

extern "C" int moe_route_quant(const void* x_bf16, const int32_t* topk_ids, int64_t T, int64_t K,
                               int64_t k, int64_t E, void* xq_u8, void* xs_u8, int32_t* sorted_row,
                               int32_t* expanded_row_idx, int64_t* group_list, void* workspace,
                               size_t ws_bytes, void* stream) {
  using namespace mxmoe;
  int rc = check_route_args(T, K, k, E);
  if (rc) return rc;
  if (!group_list || !workspace) return fail(MX_ERR_INVALID_ARG, "moe_route_quant: null pointer");
  if (T > 0 && (!x_bf16 || !topk_ids || !xq_u8 || !xs_u8 || !sorted_row || !expanded_row_idx))
    return fail(MX_ERR_INVALID_ARG, "moe_route_quant: null pointer");
  const size_t need = route_workspace_bytes(T, k, E);
  if (ws_bytes < need)
    return fail(MX_ERR_WORKSPACE, "moe_route_quant: workspace %zu bytes < %zu needed", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(x_bf16) % 16 || reinterpret_cast<uintptr_t>(xq_u8) % 16)
    return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: x and xq must be 16-byte aligned");
  return launch_route_quant(static_cast<const uint16_t*>(x_bf16), topk_ids, T, K, k, E,
                            static_cast<uint8_t*>(xq_u8), static_cast<uint8_t*>(xs_u8), sorted_row,
                            expanded_row_idx, group_list, workspace, as_stream(stream));
}

// ---------------------------------------------------------------------------
// moe_route_quant_noalloc: the same routing for callers that cannot allocate
// (code under graph capture, tight serving loops).  The only scratch the
// routing kernels use -- per-chunk expert counts, scanned in place, and the
// experts' totals -- lives in this file-scope device array instead of a
// caller workspace.  Every element the kernels read is first written by the
// same call (the histogram writes every chunk's count of every expert, the
// scan every total), so nothing needs clearing between calls; calls that
// overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------

namespace mxmoe {
constexpr size_t kRouteScratchBytes = (size_t)4 << 20;
}  // namespace mxmoe

// The routing scratch of moe_route_quant_noalloc: each GPU the library runs
// on holds its own copy until the process ends.
static __device__ __align__(256) uint8_t scratch[mxmoe::kRouteScratchBytes];

namespace mxmoe {
namespace {

std::mutex g_scratch_mutex;
void* g_scratch_dev[64] = {};

// Device address of `scratch` on the current device, looked up once per
// device (the array's name in host code is only a handle for the lookup).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MX_ERR_HIP, "moe_route_quant_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant_noalloc: device %d >= 64", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MX_ERR_HIP, "moe_route_quant_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MX_OK;
}

}  // namespace
}  // namespace mxmoe

extern "C" int moe_route_quant_noalloc(const void* x_bf16, const int32_t* topk_ids, int64_t T, int64_t K,
                                       int64_t k, int64_t E, void* xq_u8, void* xs_u8, int32_t* sorted_row,
                                       int32_t* expanded_row_idx, int64_t* group_list, void* stream) {
  using namespace mxmoe;
  int rc = check_route_args(T, K, k, E);
  if (rc) return rc;
  if (!group_list) return fail(MX_ERR_INVALID_ARG, "moe_route_quant_noalloc: null pointer");
  if (T > 0 && (!x_bf16 || !topk_ids || !xq_u8 || !xs_u8 || !sorted_row || !expanded_row_idx))
    return fail(MX_ERR_INVALID_ARG, "moe_route_quant_noalloc: null pointer");
  const size_t need = route_workspace_bytes(T, k, E);
  if (need > kRouteScratchBytes)
    return fail(MX_ERR_UNSUPPORTED,
                "moe_route_quant_noalloc: T=%lld k=%lld E=%lld needs %zu bytes of routing scratch, more than the "
                "%zu the library holds; use moe_route_quant with a workspace",
                (long long)T, (long long)k, (long long)E, need, kRouteScratchBytes);
  if (reinterpret_cast<uintptr_t>(x_bf16) % 16 || reinterpret_cast<uintptr_t>(xq_u8) % 16)
    return fail(MX_ERR_UNSUPPORTED, "moe_route_quant_noalloc: x and xq must be 16-byte aligned");
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return launch_route_quant(static_cast<const uint16_t*>(x_bf16), topk_ids, T, K, k, E,
                            static_cast<uint8_t*>(xq_u8), static_cast<uint8_t*>(xs_u8), sorted_row,
                            expanded_row_idx, group_list, ws, as_stream(stream));
}
