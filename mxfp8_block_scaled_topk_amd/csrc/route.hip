// moe_route_quant: top-k routing with the MX activation quant fused in.
//
// The T*k assignments (flat index i = t*k + j) are cut into chunks of whole
// tokens, at most 256 assignments each (one per thread).  One launch; its
// workgroups take one of three roles by block index:
//
//   leaders (blocks [0, S))  each owns a run of G consecutive chunks (a
//            super-chunk): per chunk and expert, the assignment count (LDS
//            atomics: counts are order-free, so atomics keep them exact),
//            stored as the exclusive prefix over the super-chunk's earlier
//            chunks, plus the super-chunk's total per expert; then the call's
//            tag goes into the leader's flag.  Block 0 then also waits for
//            every leader's flag and sets one ready flag.
//   scatter  the rest: each owns a share of one chunk's tokens.  It finds the
//            stable rank of every assignment of the chunk among those to the
//            same expert (wave ballot match + per-wave counts in LDS) and
//            MX-quantises its share into LDS (two lanes per 32-element block,
//            the block's amax combined with one lane exchange); only then
//            does it wait for the ready flag, so the activation reads of the
//            workgroups resident at the start overlap the counting.  It then
//            loads the S x E super-chunk totals and scans them itself: an
//            expert's total (the first share of chunk 0 writes group_list),
//            its row offset (exclusive scan over the experts) and its count
//            before this super-chunk.  Row p = expert offset + super-chunk
//            prefix + chunk prefix + rank; the first share of a chunk writes
//            both maps; each quantised row then goes from LDS to the token's
//            k rows, 16 bytes per lane, whole lines per store instruction.
//            Shares are sized so that a share's rows fit a 40 KB LDS budget
//            and the grid holds at least four workgroups per compute unit (at
//            the 16K prefill size: two shares of 16 tokens, 1024 workgroups,
//            all resident at once).  Most of the traffic is HBM writes (k
//            quantised copies of every token).
//
// Flags hold a 64-bit tag unique to the call, so the workspace needs no
// clearing: a flag left by an earlier call never matches.  Every wait is
// bounded: a block whose wait runs out (the leaders not yet scheduled, or a
// test forcing it) counts what it needs from topk_ids itself -- the same
// integers, so the output does not depend on which path a block took, and
// the kernel ends whatever order the hardware runs its workgroups in.
//
// When all T*k assignments fit in one chunk (decode-sized batches) there are
// no leaders: the scatter blocks take the experts' totals from their own
// per-wave counts, and the first block writes the group list.
//
// The order inside an expert is the flat index order, so the permutation is
// deterministic and equals a stable sort by expert.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>

#include <unistd.h>

#include "common.h"

namespace mxmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 1024;
// most leader blocks (super-chunks) per call
constexpr int kMaxLeaders = 32;
// the routing workspace's control block: the 64-bit generation word
constexpr size_t kCtrlBytes = 256;
// LDS a scatter workgroup may fill with its share's quantised rows
constexpr int kXBufBytes = 40 << 10;
// scatter workgroups wanted per compute unit (a chunk is split into more
// shares until the grid has that many)
constexpr int kScatterPerCU = 4;
// shares of a single-chunk batch (decode sizes) unless the LDS budget needs
// more (such calls are launch-bound: 16 or 32 shares time the same)
constexpr int kSingleShares = 16;

struct RouteParams {
  const uint16_t* x;
  const int32_t* ids;
  uint8_t* xq;
  uint8_t* xs;
  int32_t* sorted_row;
  int32_t* eri;
  int64_t* group_list;
  int32_t* chunk_pre;   // [nch][E] count prefix over the super-chunk's earlier chunks
  int32_t* super;       // [S][E] super-chunk totals per expert
  uint64_t* flags;      // [S + 1]: one per leader, then the ready flag
  const uint64_t* gen;  // the workspace's generation word (see call_tag)
  uint64_t tag;         // unique to the host call (the flags' tag mixes in *gen)
  int64_t wait_limit;   // polls before a block counts for itself
  int64_t T, K;
  int k, E, nbits, tpc, nch, G, S;
  int split;            // scatter workgroups (shares) per chunk
  int nbuf;             // tokens of a share quantised into LDS before the wait
  int row_bytes;        // LDS bytes per such token: K payload, then the scales, padded to 16
  int lds_ints;         // dynamic LDS of the launch, in ints
  int scales16;         // xs rows can be written 16 bytes at a time
};

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

__device__ __forceinline__ uint64_t load_flag(const uint64_t* f) {
  return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls *f until it holds `tag`, at most `limit` times; true if it did.
__device__ bool wait_flag(const uint64_t* f, uint64_t tag, int64_t limit) {
  for (int64_t n = 0; n < limit; ++n) {
    if (load_flag(f) == tag) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Cross-workgroup exchange.  Everything one workgroup publishes to another
// (counts and flags) is written and read with device-scope accesses
// (agent-scope atomics: loads and stores carrying the device scope bits), which
// go to the device's coherence point instead of a compute unit's or an XCD's
// own cache.  A publisher waits until its device-scope stores are complete
// (s_waitcnt vmcnt(0): on this architecture the counter covers stores), meets
// the block barrier, and only then sets the flag; a reader polls the flag,
// meets its block barrier, and only then issues its loads.  So a reader that
// sees the call's tag reads the values stored before it.  This takes the place
// of release and acquire fences at agent scope, which write back and
// invalidate the whole L2 of the XCD: measured at about 7 us per publishing
// workgroup (the L2 still holds the previous kernel's dirty lines), and more
// than the routing's own traffic when every scatter workgroup invalidates.
__device__ __forceinline__ int load_coherent(const int32_t* q) {
  return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int32_t* q, int v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The tag this launch's flags carry: the host call's tag mixed with the
// workspace's generation word.  A call made under stream capture records a
// kernel that advances the generation before the routing kernel, so every
// replay of the captured work has its own tag although its arguments, the
// host tag included, are the captured ones.
__device__ __forceinline__ uint64_t call_tag(const RouteParams& p, uint64_t gen) {
  return p.tag ^ (gen * 0x9E3779B97F4A7C15ull);
}

// Publishes the block's earlier device-scope stores under flag *f.
__device__ void publish(uint64_t* f, uint64_t tag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt not waited for
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(f, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-expert counts of the valid assignments in [0, M) into tot[0..E), and of
// those with flat index below `before` into pre[0..E) (pre may be null).
__device__ void count_all(const RouteParams& p, int64_t before, int* tot, int* pre) {
  for (int e = threadIdx.x; e < p.E; e += kThreads) {
    tot[e] = 0;
    if (pre) pre[e] = 0;
  }
  __syncthreads();
  const int64_t M = p.T * p.k;
  for (int64_t i = threadIdx.x; i < M; i += kThreads) {
    const int e = p.ids[i];
    if (e < 0 || e >= p.E) continue;
    atomicAdd(&tot[e], 1);
    if (pre && i < before) atomicAdd(&pre[e], 1);
  }
  __syncthreads();
}

// Leader of super-chunk s: chunks [s*G, min((s+1)*G, nch)).
__device__ void leader(const RouteParams& p, int s, int* smem, int lds_ints, uint64_t tag) {
  const int tid = threadIdx.x, E = p.E;
  const int per_chunk = p.tpc * p.k;   // assignments per full chunk (<= 256)
  const int64_t M = p.T * p.k;
  const int c0 = s * p.G, c1 = std::min(c0 + p.G, p.nch);
  int* run = smem;             // [E] running count over the super-chunk
  int* hist = smem + E;        // [gb][E] counts of a batch of chunks
  const int gb = lds_ints / E - 1;   // chunks per batch (>= 3)
  for (int e = tid; e < E; e += kThreads) run[e] = 0;
  for (int cb = c0; cb < c1; cb += gb) {
    const int nb = std::min(gb, c1 - cb);
    for (int i = tid; i < nb * E; i += kThreads) hist[i] = 0;
    __syncthreads();
    if (tid < per_chunk) {
      constexpr int kU = 16;   // loads in flight per thread
      for (int j0 = 0; j0 < nb; j0 += kU) {
        int ev[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t a = (int64_t)(cb + j0 + u) * per_chunk + tid;
          ev[u] = (j0 + u < nb && a < M) ? p.ids[a] : -1;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (ev[u] >= 0 && ev[u] < E) atomicAdd(&hist[(j0 + u) * E + ev[u]], 1);
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      int r = run[e];
      for (int j = 0; j < nb; ++j) {
        store_coherent(&p.chunk_pre[(int64_t)(cb + j) * E + e], r);
        r += hist[j * E + e];
      }
      run[e] = r;
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += kThreads) store_coherent(&p.super[(int64_t)s * E + e], run[e]);
  publish(&p.flags[s], tag);
}

// MX quant of one half of a 32-element block (16 bf16 in u0, u1); the other
// half sits in the neighbouring lane (lane ^ 1), which must be active.
__device__ __forceinline__ void quant_half_regs(const uint4& u0, const uint4& u1, uint4& q, uint32_t& sb) {
  float v[16];
  unpack_bf16x8(u0, v);
  unpack_bf16x8(u1, v + 8);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  sb = e8m0_from_amax(amax);
  const float inv = e8m0_inverse(sb);
  q.x = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  q.y = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  q.z = e4m3x4(v[8] * inv, v[9] * inv, v[10] * inv, v[11] * inv);
  q.w = e4m3x4(v[12] * inv, v[13] * inv, v[14] * inv, v[15] * inv);
}

__device__ __forceinline__ void quant_half_block(const RouteParams& p, int64_t t, int b, int half, uint4& q,
                                                 uint32_t& sb) {
  const uint4* src = reinterpret_cast<const uint4*>(p.x + t * p.K + (b * 32 + half * 16));
  quant_half_regs(src[0], src[1], q, sb);
}

// kSingle: all assignments in one chunk (no leaders, no waits).
template <bool kSingle>
__global__ __launch_bounds__(kThreads) void route_quant_kernel(RouteParams p) {
  // dynamic LDS: [4E ints: per-wave expert counts, or a leader's chunk counts
  // (its whole LDS)] [kThreads ints: s_pos] [the share's quantised rows,
  // row_bytes each]
  extern __shared__ __align__(16) int dyn[];
  __shared__ int s_wsum[kThreads / 64];
  __shared__ uint64_t s_gen;   // the workspace's generation word, read once by thread 0

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E;
  if (!kSingle && (int)blockIdx.x < p.S) {   // uniform per block
    if (tid == 0) s_gen = __hip_atomic_load(p.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint64_t tag = call_tag(p, s_gen);
    leader(p, blockIdx.x, dyn, p.lds_ints, tag);
    if (blockIdx.x == 0) {
      // gather the leaders' flags into the one flag the scatter workgroups
      // poll (left unset if a leader has not finished in time: the scatter
      // workgroups then count for themselves)
      bool ok = true;
      if (tid < p.S) ok = wait_flag(&p.flags[tid], tag, p.wait_limit);
      if (__syncthreads_and(ok) && tid == 0)
        __hip_atomic_store(&p.flags[p.S], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  constexpr bool single = kSingle;
  int* s_wcnt = dyn;                 // [4][E]
  int* s_pos = dyn + 4 * E;          // [kThreads]
  uint8_t* xbuf = reinterpret_cast<uint8_t*>(dyn + 4 * E + kThreads);
  const int64_t M = p.T * p.k;
  const int nb = (int)(p.K / 32);      // K <= 2^24: every in-row index below fits 32 bits
  const int s_stride = ((nb + 1) / 2) * 2;
  const int hpr = 2 * nb;              // half-blocks per token row
  int ready = single ? 1 : -1;   // block-uniform: -1 not yet waited, 1 counts published, 0 count here

  const int64_t w = (int64_t)blockIdx.x - p.S;   // (chunk c, share `part` of its tokens)
  const int c = (int)(w / p.split), part = (int)(w % p.split);
  for (int i = tid; i < 4 * E; i += kThreads) s_wcnt[i] = 0;
  __syncthreads();

  // ---- stable rank of each assignment within the chunk -------------------
  // (thread 0 also looks at the ready flag, in the same memory round trip as
  // the ids)
  bool seen = true;
  uint64_t tag = 0;
  if (!single && tid == 0) {
    const uint64_t g = __hip_atomic_load(p.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t f = load_flag(&p.flags[p.S]);
    tag = call_tag(p, g);
    seen = f == tag;
  }
  const int64_t a0 = (int64_t)c * p.tpc * p.k;
  const int na = (int)std::min<int64_t>((int64_t)p.tpc * p.k, M - a0);
  const int64_t a = a0 + tid;
  int e = 0;
  bool valid = false;
  if (tid < na) {
    e = p.ids[a];
    valid = e >= 0 && e < E;
  }
  uint64_t same = __ballot(valid);
  for (int bit_i = 0; bit_i < p.nbits; ++bit_i) {
    const bool bit = valid && ((e >> bit_i) & 1);
    const uint64_t ones = __ballot(bit);
    same &= bit ? ones : ~ones;
  }
  int rank = __popcll(same & ((1ull << lane) - 1ull));
  if (valid && rank == 0) s_wcnt[wave * E + e] = __popcll(same);
  if (__syncthreads_and(seen)) ready = 1;   // uniform; always true for a single chunk
  if (valid)
    for (int wv = 0; wv < wave; ++wv) rank += s_wcnt[wv * E + e];

  // ---- this share's tokens: the first nbuf quantised into LDS now ---------
  const int64_t t0 = (int64_t)c * p.tpc;   // the share's tokens: [tb, te) of the chunk
  const int ntok = (int)std::min<int64_t>((int64_t)p.tpc, p.T - t0);
  const int per = (p.tpc + p.split - 1) / p.split;
  const int tb = std::min(part * per, ntok), te = std::min(tb + per, ntok);
  const int nbt = std::min(te - tb, p.nbuf);
  const int rowb = p.row_bytes;   // payload K bytes, then s_stride scale bytes, padded to 16
  const int n_it = nbt * hpr;     // half-blocks; even, so lane pairs stay together
  constexpr int kLd = 4;          // half-blocks whose loads a lane has in flight at once
  for (int it0 = tid; it0 < n_it; it0 += kLd * kThreads) {
    uint4 u[kLd][2];
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int it = it0 + i * kThreads;
      if (it < n_it) {
        const int tl = it / hpr, hb = it - tl * hpr;
        const uint4* src = reinterpret_cast<const uint4*>(p.x + (t0 + tb + tl) * p.K + (hb * 16));
        u[i][0] = src[0];
        u[i][1] = src[1];
      }
    }
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int it = it0 + i * kThreads;
      if (it < n_it) {
        const int tl = it / hpr, hb = it - tl * hpr;
        uint4 q;
        uint32_t sb;
        quant_half_regs(u[i][0], u[i][1], q, sb);
        uint8_t* row = xbuf + tl * rowb;
        *reinterpret_cast<uint4*>(row + hb * 16) = q;
        if ((hb & 1) == 0) {
          row[p.K + (hb >> 1)] = static_cast<uint8_t>(sb);
          if ((nb & 1) && (hb >> 1) == nb - 1) row[p.K + nb] = 0;
        }
      }
    }
  }

  // ---- row of each assignment --------------------------------------------
  int pos = -1;
  if (single) {
    // the only chunk's counts are the experts' totals; s_tot overwrites the
    // last per-wave row only after every wave has read it (barrier below)
    int* s_tot = s_wcnt + 3 * E;
    int cnt[kMaxE / kThreads];
#pragma unroll
    for (int i = 0; i < kMaxE / kThreads; ++i) {
      const int ee = tid + i * kThreads;
      int n = 0;
      if (ee < E)
        for (int wv = 0; wv < kThreads / 64; ++wv) n += s_wcnt[wv * E + ee];
      cnt[i] = n;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxE / kThreads; ++i) {
      const int ee = tid + i * kThreads;
      if (ee < E) {
        s_tot[ee] = cnt[i];
        if (part == 0) p.group_list[ee] = cnt[i];
      }
    }
    __syncthreads();
    block_exclusive_scan(s_tot, E, s_tot, s_wsum);
    __syncthreads();
    if (valid) pos = s_tot[e] + rank;
  } else {
    if (ready < 0) {
      // thread 0 polls the ready flag; the barrier orders every wave's count
      // loads after it was seen
      bool ok = true;
      if (tid == 0) ok = wait_flag(&p.flags[p.S], tag, p.wait_limit);   // thread 0 holds the tag
      ready = __syncthreads_and(ok) ? 1 : 0;
    } else {
      __syncthreads();   // the per-wave counts are read: their LDS is reused below
    }
    if (ready) {
      // every expert's total and its count before this chunk's super-chunk,
      // from the leaders' counts; the expert offsets by a scan over E
      int* tot = s_wcnt;
      int* pre = s_wcnt + E;
      int* off = s_wcnt + 2 * E;
      const int sc = c / p.G;
      const int S = p.S;
      int cp = 0;
      if (valid) cp = load_coherent(&p.chunk_pre[(int64_t)c * E + e]);
      for (int e2 = tid; e2 < E; e2 += kThreads) {
        int t = 0, b = 0;
        constexpr int kU = 16;   // loads in flight (index clamped to S-1, the surplus discarded)
        for (int j0 = 0; j0 < S; j0 += kU) {
          int v[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) v[u] = load_coherent(&p.super[(int64_t)std::min(j0 + u, S - 1) * E + e2]);
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            t += j0 + u < S ? v[u] : 0;
            b += j0 + u < sc ? v[u] : 0;
          }
        }
        tot[e2] = t;
        pre[e2] = b;
      }
      __syncthreads();
      block_exclusive_scan(tot, E, off, s_wsum);
      __syncthreads();
      if (c == 0 && part == 0)
        for (int e2 = tid; e2 < E; e2 += kThreads) p.group_list[e2] = tot[e2];
      if (valid) pos = off[e] + pre[e] + cp + rank;
    } else {
      // count for this chunk here: every expert's total and its count
      // before the chunk, from topk_ids (the per-wave counts are done with)
      __syncthreads();
      int* tot = s_wcnt;
      int* pre = s_wcnt + E;
      int* off = s_wcnt + 2 * E;
      count_all(p, a0, tot, pre);
      block_exclusive_scan(tot, E, off, s_wsum);
      __syncthreads();
      if (c == 0 && part == 0)
        for (int e2 = tid; e2 < E; e2 += kThreads) p.group_list[e2] = tot[e2];
      if (valid) pos = off[e] + pre[e] + rank;
    }
  }
  if (valid && part == 0) p.sorted_row[pos] = (int32_t)a;
  if (part == 0 && tid < na) p.eri[a] = pos;
  s_pos[tid] = pos;
  __syncthreads();   // s_pos and the LDS rows are complete

  // ---- stores: each buffered row to the token's k rows ---------------------
  const int k = p.k;
  const int n16 = (int)(p.K / 16);   // 16-byte pieces of a payload row
  for (int idx = tid; idx < nbt * k * n16; idx += kThreads) {
    const int rowi = idx / n16, ch = idx - rowi * n16;
    const int tl = rowi / k, j = rowi - tl * k;
    const int r = s_pos[(tb + tl) * k + j];
    if (r < 0) continue;
    *reinterpret_cast<uint4*>(p.xq + (int64_t)r * p.K + ch * 16) =
        *reinterpret_cast<const uint4*>(xbuf + tl * rowb + ch * 16);
  }
  if (p.scales16) {
    const int s16 = s_stride / 16;
    for (int idx = tid; idx < nbt * k * s16; idx += kThreads) {
      const int rowi = idx / s16, ch = idx - rowi * s16;
      const int tl = rowi / k, j = rowi - tl * k;
      const int r = s_pos[(tb + tl) * k + j];
      if (r < 0) continue;
      *reinterpret_cast<uint4*>(p.xs + (int64_t)r * s_stride + ch * 16) =
          *reinterpret_cast<const uint4*>(xbuf + tl * rowb + p.K + ch * 16);
    }
  } else {
    for (int idx = tid; idx < nbt * k * s_stride; idx += kThreads) {
      const int rowi = idx / s_stride, ch = idx - rowi * s_stride;
      const int tl = rowi / k, j = rowi - tl * k;
      const int r = s_pos[(tb + tl) * k + j];
      if (r < 0) continue;
      p.xs[(int64_t)r * s_stride + ch] = xbuf[tl * rowb + p.K + ch];
    }
  }

  // ---- the share's tokens past the LDS budget: quantised and stored here ---
  for (int it = nbt * hpr + tid; it < (te - tb) * hpr; it += kThreads) {
    const int tl = tb + it / hpr;
    const int hb = it - (tl - tb) * hpr;
    const int b = hb >> 1;
    const int half = hb & 1;
    uint4 q;
    uint32_t sb;
    quant_half_block(p, t0 + tl, b, half, q, sb);
    for (int j = 0; j < k; ++j) {
      const int r = s_pos[tl * k + j];
      if (r < 0) continue;
      *reinterpret_cast<uint4*>(p.xq + (int64_t)r * p.K + (b * 32 + half * 16)) = q;
      if (half == 0) {
        p.xs[(int64_t)r * s_stride + b] = static_cast<uint8_t>(sb);
        if ((nb & 1) && b == nb - 1) p.xs[(int64_t)r * s_stride + nb] = 0;
      }
    }
  }
}

// Advances a routing workspace's generation word (recorded before the
// routing kernel when the stream is capturing).
__global__ void bump_generation(uint64_t* gen) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *gen += 1;
}

__global__ void zero_i64(int64_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

struct Split {
  int64_t tpc, nch, G, S;
};

// Chunks and super-chunks of a call (S = 0 when one chunk holds everything).
inline Split split_of(int64_t T, int64_t k) {
  Split s;
  s.tpc = std::max<int64_t>(1, kThreads / k);
  s.nch = (T + s.tpc - 1) / s.tpc;
  if (s.nch <= 1) {
    s.G = 1;
    s.S = 0;
  } else {
    s.G = (s.nch + kMaxLeaders - 1) / kMaxLeaders;
    s.S = (s.nch + s.G - 1) / s.G;
  }
  return s;
}

// 64-bit tags unique to each launch in this process: a random 32-bit process
// salt (never 0) over a 32-bit launch counter.
uint64_t next_tag() {
  static const uint64_t salt = [] {
    uint64_t v = (uint64_t)getpid() ^ ((uint64_t)getpid() << 40) ^
                 (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    try {
      std::random_device rd;
      v ^= ((uint64_t)rd() << 32) ^ rd();
    } catch (...) {
      // no entropy source: the process id and the clock alone
    }
    v = (v ^ (v >> 32)) & 0xffffffffull;
    return v ? v : 0x9e3779b9ull;
  }();
  static std::atomic<uint32_t> counter{0};
  return (salt << 32) | (uint64_t)counter.fetch_add(1, std::memory_order_relaxed);
}

std::atomic<int64_t> g_wait_limit{(int64_t)1 << 18};


}  // namespace

size_t route_workspace_bytes(int64_t T, int64_t k, int64_t E) {
  const Split s = split_of(T, k);
  if (s.S == 0) return 0;
  return kCtrlBytes + align_up((size_t)(E * s.nch) * 4, 256) + align_up((size_t)(E * s.S) * 4, 256) +
         align_up((size_t)(s.S + 1) * 8, 256);
}

int check_route_args(int64_t T, int64_t K, int64_t k, int64_t E) {
  if (T < 0 || K <= 0 || k <= 0 || E <= 0)
    return fail(MX_ERR_INVALID_ARG, "moe_route_quant: bad sizes T=%lld K=%lld k=%lld E=%lld",
                (long long)T, (long long)K, (long long)k, (long long)E);
  if (k > E) return fail(MX_ERR_INVALID_ARG, "moe_route_quant: k=%lld > E=%lld", (long long)k, (long long)E);
  if (!dims_in_range({T, K})) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: T or K above 2^31 - 1");
  if (K % 32 != 0) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: K=%lld is not a multiple of 32", (long long)K);
  if (K > (int64_t)1 << 24) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: K=%lld > 2^24", (long long)K);
  if (k > kThreads) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: k=%lld > %d", (long long)k, kThreads);
  if (E > kMaxE) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: E=%lld > %d", (long long)E, kMaxE);
  // the launch holds 16 workgroups of 256 threads per 256 assignments, and a
  // grid holds fewer than 2^32 threads
  if (T * k > (int64_t)1 << 27) return fail(MX_ERR_UNSUPPORTED, "moe_route_quant: T*k > 2^27");
  return MX_OK;
}

int launch_route_quant(const uint16_t* x, const int32_t* ids, int64_t T, int64_t K, int64_t k,
                       int64_t E, uint8_t* xq, uint8_t* xs, int32_t* sorted_row, int32_t* eri,
                       int64_t* group_list, void* ws, hipStream_t stream) {
  if (T == 0) {
    zero_i64<<<dim3((unsigned)((E + 255) / 256)), dim3(256), 0, stream>>>(group_list, (int)E);
    return check_launch("moe_route_quant(zero)");
  }
  const Split sp = split_of(T, k);
  RouteParams p{};
  p.x = x;
  p.ids = ids;
  p.xq = xq;
  p.xs = xs;
  p.sorted_row = sorted_row;
  p.eri = eri;
  p.group_list = group_list;
  if (sp.S > 0) {
    char* w = static_cast<char*>(ws);
    p.gen = reinterpret_cast<const uint64_t*>(w);
    w += kCtrlBytes;
    const size_t pre_bytes = align_up((size_t)(E * sp.nch) * 4, 256);
    p.chunk_pre = reinterpret_cast<int32_t*>(w);
    p.super = reinterpret_cast<int32_t*>(w + pre_bytes);
    p.flags = reinterpret_cast<uint64_t*>(w + pre_bytes + align_up((size_t)(E * sp.S) * 4, 256));
  }
  p.tag = next_tag();
  p.wait_limit = g_wait_limit.load(std::memory_order_relaxed);
  p.T = T;
  p.K = K;
  p.k = (int)k;
  p.E = (int)E;
  int nbits = 0;
  while ((1ll << nbits) < E) ++nbits;
  p.nbits = nbits;
  p.tpc = (int)sp.tpc;
  p.nch = (int)sp.nch;
  p.G = (int)sp.G;
  p.S = (int)sp.S;
  // shares per chunk: doubled until a share's quantised rows fit the LDS
  // budget and the grid has kScatterPerCU workgroups per compute unit (at
  // most one token per share); a batch of one chunk (nothing to wait for)
  // takes at most kSingleShares
  const int64_t nb = K / 32, s_stride = ((nb + 1) / 2) * 2;
  const int64_t row_bytes = (int64_t)align_up((size_t)(K + s_stride), 16);
  const int64_t want = sp.S == 0 ? kSingleShares : (int64_t)num_cus() * kScatterPerCU;
  int64_t split = 1;
  while (split < sp.tpc &&
         (((sp.tpc + split - 1) / split) * row_bytes > kXBufBytes || sp.nch * split < want))
    split *= 2;
  split = std::min(split, sp.tpc);
  const int64_t per = (sp.tpc + split - 1) / split;
  p.split = (int)split;
  p.nbuf = (int)std::min<int64_t>(per, kXBufBytes / row_bytes);
  p.row_bytes = (int)row_bytes;
  const size_t lds = (size_t)(4 * E + kThreads) * 4 + (size_t)p.nbuf * (size_t)row_bytes;
  p.lds_ints = (int)(lds / 4);
  p.scales16 = (reinterpret_cast<uintptr_t>(xs) % 16 == 0 && s_stride % 16 == 0) ? 1 : 0;
  const int64_t grid = sp.S + sp.nch * split;
  if (sp.S == 0) {
    route_quant_kernel<true><<<dim3((unsigned)grid), dim3(kThreads), lds, stream>>>(p);
  } else {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
      return fail(MX_ERR_HIP, "moe_route_quant: hipStreamIsCapturing failed");
    if (cs == hipStreamCaptureStatusActive) {
      bump_generation<<<dim3(1), dim3(64), 0, stream>>>(static_cast<uint64_t*>(ws));
      const int rc = check_launch("moe_route_quant(generation)");
      if (rc) return rc;
    }
    route_quant_kernel<false><<<dim3((unsigned)grid), dim3(kThreads), lds, stream>>>(p);
  }
  return check_launch("route_quant_kernel");
}

}  // namespace mxmoe

extern "C" int64_t moe_route_quant_set_wait_limit(int64_t polls) {
  return mxmoe::g_wait_limit.exchange(polls < 0 ? 0 : polls);
}

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
  const size_t need = route_workspace_bytes(T, k, E);
  if (!group_list || (need > 0 && !workspace)) return fail(MX_ERR_INVALID_ARG, "moe_route_quant: null pointer");
  if (T > 0 && (!x_bf16 || !topk_ids || !xq_u8 || !xs_u8 || !sorted_row || !expanded_row_idx))
    return fail(MX_ERR_INVALID_ARG, "moe_route_quant: null pointer");
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
// routing kernel uses -- the generation word, per-chunk expert counts, the
// super-chunk totals and the flags that publish them -- lives in this
// file-scope device array instead of a caller workspace.  Every count the
// kernel reads is first written by the same call, and a flag matches only the
// tag of the call (or graph replay) that set it, so nothing needs clearing
// between calls; calls that overlap on one GPU share the array and race.
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
