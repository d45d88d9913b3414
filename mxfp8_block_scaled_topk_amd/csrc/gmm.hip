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
// Tiling.  A workgroup of 8 waves (two per SIMD) computes a 256 (weight
// rows) x 256 (tokens) tile; wave w computes a 128 x 64 part (rows
// 128*(w%2), tokens 64*(w/2)) as 4 x 2 MFMA tiles, 128 fp32 accumulators per
// lane.  When the experts average few rows (decode-sized batches) the same
// kernel runs 256 x 128-token tiles with a three-slot ring (see kBM).
//
// Data movement.  K advances 128 bytes per stage through a two-slot LDS ring
// (66 KB per slot: 256 rows x 128 B of each operand plus the u32 of 4 scale
// bytes per row), filled by direct global->LDS loads (global_load_lds_dwordx4
// / _dword, 1 KB per instruction, no staging registers).  When the k stages
// divide into groups of 4, the scales instead come 16 bytes per row (4
// stages) at a time into a small double-buffered ring of their own: a scale
// row is 1/32 of an operand row, so per-stage dword loads touch a line for
// every two rows and made up a third of all line requests.  Whole 128-byte rows
// matter: measured on gfx950, 64-byte row pieces halve the L2->LDS rate.  The
// loads are issued from inline assembly with explicit vmcnt accounting (the
// compiler otherwise waits for every outstanding LDS DMA before any LDS
// read).  Each DMA takes a uniform 64-bit base in scalar registers and a
// 32-bit per-lane offset.  The 16-byte chunk index of a row is XOR-ed with
// (row/2)%8: the 16 lanes of one 256-byte LDS access (consecutive rows, one
// chunk column) then hit 16 distinct 4-bank groups of the 64-bank LDS; the
// swizzle is applied on the global side by choosing which chunk each DMA
// lane fetches.
//
// Pipeline.  A stage is two 64-wide k sub-steps of 8 MFMAs per wave.  Each
// operand fragment is reloaded from LDS for the next sub-step right after its
// last MFMA, so the LDS reads overlap the matrix work (measured: with reads
// grouped ahead of the MFMAs the two waves of a SIMD ran in lockstep and the
// MFMA pipe idled while both waited).  One barrier per stage sits between
// the two sub-steps; after it the slot of the current stage is free and the
// DMA for the stage after next goes into it, a full stage ahead of its use.
// At the current sizes moving the operands is what bounds the kernel, mostly
// through the clock it costs under the power limit (measured at the 16K
// prefill size: without the operand DMA the shader clock rises from about
// 1.86 to 2.2 GHz and the GEMMs run 15-25 % faster; with every operand an L2
// hit, 6 % (GEMM1) and 16 % (GEMM2) faster).
//
// Scheduling.  The kernel is persistent (one workgroup per CU).  Every
// workgroup derives the per-expert row ranges and m-tile prefix from the
// device-resident group list (no host synchronisation).  Tile t is m-tile
// t / n_tiles (an m-tile never straddles two experts) and n-tile t % n_tiles;
// workgroups are dealt to the 8 XCDs round-robin and each XCD's CUs walk
// neighbouring tiles (see the tile walk in the kernel), so operands are
// shared in that XCD's L2.  The stage stream runs across tile boundaries.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace mxmoe {

namespace {

constexpr int BM = 256;  // token rows per tile (the 128-row variant: kBM below)
constexpr int BN = 256;  // weight rows per tile
constexpr int BK = 128;  // K bytes per stage
constexpr int kThreads = 512;
constexpr int kMaxE = 1024;
constexpr int64_t kMaxKd = (int64_t)1 << 20;   // reduction size limit (32-bit DMA offsets)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
// LDS reads the compiler must leave where they are written (between the MFMAs
// they overlap): volatile, so no IR pass hoists them.
typedef __attribute__((address_space(3))) const volatile u32x4 lds_u32x4_v;
typedef __attribute__((address_space(3))) const volatile uint8_t lds_u8_v;

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

constexpr int SK = 128;          // K bytes per stage (whole 128-byte rows)

// One ring slot: a k stage of both operands for a tile of kRows token rows,
// and with per-stage scale loads (kScales) the stage's scale word of every
// row (4 bytes: its four 32-blocks).
template <int kRows, bool kScales>
struct StageT {
  uint8_t a[BN * SK];
  uint8_t b[kRows * SK];
  uint32_t sa[BN];
  uint32_t sb[kRows];
};
template <int kRows>
struct StageT<kRows, false> {
  uint8_t a[BN * SK];
  uint8_t b[kRows * SK];
};

// Group-list types: 0 cumulative, 1 counts (the entry points' two forms);
// 2, used only inside the library (the dense linear), one group holding all
// M rows with no list in memory.
constexpr int kGlSingle = 2;
__device__ __forceinline__ int64_t group_count(const int64_t* gl, int type, int e, int64_t M) {
  if (type == kGlSingle) return e == 0 ? M : 0;
  if (type == 1) return gl[e];
  return gl[e] - (e > 0 ? gl[e - 1] : 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// 64 lanes x 16 B from global (uniform base + per-lane 32-bit offset) to LDS
// [m0, m0 + 1024).
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// 64 lanes x 4 B to LDS [m0, m0 + 256).
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// s_waitcnt vmcnt(n) for a wave-uniform n (vmcnt(0) above 7): every VMEM
// instruction but the n latest has completed
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
// Workgroup barrier that first drains this wave's LDS reads, so no read of a
// slot can still be pending when the next DMA into that slot is issued.
__device__ __forceinline__ void barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// The same value, opaque to the optimiser: address arithmetic derived from it
// is done where it is used instead of being hoisted out of the tile loop
// (which would keep dozens of per-lane addresses live through the k loop).
__device__ __forceinline__ int opaque(int v) {
  asm("" : "+v"(v));
  return v;
}
// A value the whole wave agrees on, moved to scalar registers.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ const T* uniptr(const T* p) {
  return reinterpret_cast<const T*>(uni64(reinterpret_cast<int64_t>(p)));
}

// Two floats -> two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// silu(g) * u with the hardware exp and reciprocal (about 1 ulp each).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Where one workgroup's tile lives.
struct TileInfo {
  int e, nt;
  int64_t m0;
  int rows_valid;
};

// Physical 16-byte chunk of logical chunk c in tile row r (128-byte rows).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// kWF: the weights' format and layout.  kWfE4m3: e4m3 rows [E, Nw, Kd].
// kWfE2m1: MXFP4 (packed e2m1, Kd/2 bytes per row, the W4A8 path); the
// token operand stays MXFP8.  kWfPacked: e4m3 in the tile-packed layout of
// mx_pack_weights -- for every (expert, n-tile, k stage) the 256 x 128
// bytes a workgroup's ring slot receives, stored contiguously in the slot's
// own row order with each row's 16-byte chunks already swizzled, so a
// stage's weight DMA reads one contiguous 32 KB block.
// kG: k stages per scale load.  kG = 1: every stage's DMA brings the 4 scale
// bytes per row of that stage (a 64-lane dword load touches 32 lines for
// 256 bytes).  kG = 4 (k stages a multiple of 4, scale rows 16-byte
// aligned): the first stage of each group of 4 brings 16 bytes per row into
// a separate double-buffered scale ring, a quarter of the line requests
// (measured: scale requests cost GEMM1 about a tenth of its time at kG = 1).
// kBM: token rows per tile.  256: the two-slot ring above.  128 (few rows
// per expert, e.g. decode batches, where the weight stream is latency-bound
// rather than MFMA-bound): each wave holds one 32-token fragment, a slot is
// 48 KB (49.5 KB with per-stage scale words), and three slots give the DMA
// two stages of lead; at least 3 k stages.  The scale ring then holds 256
// weight rows and 128 token rows per group (12 KB for both buffers), which
// fits beside the three slots while the per-expert tables, sized to E in the
// dynamic LDS, take at most 4 KB (E <= 511, host).
template <bool kSwiglu, int kWF, int kG, int kBM>
__global__ __launch_bounds__(kThreads) void gmm_kernel(GmmParams p) {
  constexpr bool kW4 = kWF == kWfE2m1;
  constexpr bool kPk = kWF == kWfPacked;
  static_assert(kG == 1 || kG == 4, "scale groups of 1 or 4 stages");
  static_assert(kBM == 256 || kBM == 128, "256- or 128-row tiles");
  constexpr int kSl = kBM == 256 ? 2 : 3;   // LDS ring slots
  constexpr int kNB = kBM / 128;            // 32-token B fragments per wave
  constexpr int kTokRows = kBM / 8;         // token rows each wave's DMA fetches
  constexpr int kNT = kTokRows / 8;         // token DMAs per wave per stage
  constexpr int kNA = kW4 ? 2 : 4;          // weight DMAs per wave per stage
  constexpr int kDmaOps = kNA + kNT + 1;    // + 1 scale load
  constexpr int kRowA = kW4 ? SK / 2 : SK;  // weight bytes per LDS row per stage
  using Stage = StageT<kBM, kG == 1>;
  __shared__ __attribute__((aligned(16))) Stage st[kSl];
  // kG = 4: scale words of 4 consecutive stages; group buffer (g/4)%2 holds
  // 256 weight rows then kBM token rows, 16 bytes per row
  constexpr uint32_t kScBuf = (BN + kBM) * 16;   // bytes per group buffer
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[kG == 4 ? 2 * kScBuf / 4 : 4];
  // per-expert tables (E + 1 ints each) in the dynamic LDS, sized by the launch
  extern __shared__ int s_tab[];
  int* const s_tile0 = s_tab;
  int* const s_row0 = s_tab + (p.E + 1);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = p.E;

  // ---- per-expert row ranges and m-tile prefix (wave 0) -------------------
  if (wave == 0) {
    constexpr int PER = kMaxE / 64;
    int64_t n[PER];
    int64_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      int64_t v = e < E ? group_count(p.group_list, p.gl_type, e, p.M) : 0;
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
      tiles[i] = (int)((r1 - r0 + kBM - 1) / kBM);
      if (e < E) s_row0[e] = (int)r0;
      if (e == E - 1) s_row0[E] = (int)r1;
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
  const int nk = (int)(Kd / SK); // stages per tile
  const int G = gridDim.x;       // a multiple of 8 (host)
  // Tile walk.  Workgroups are dealt to the 8 XCDs round-robin, so XCD x
  // holds workgroups x, x+8, ...; its 32 CUs walk the tile list with stride
  // TS from their first tile.  GEMM1: XCD x owns the contiguous eighth
  // [x*total/8, (x+1)*total/8) of the (expert, m-tile, n-tile) list, so an
  // expert's weights stay in one XCD's L2 across rounds.  GEMM2: rounds of
  // 32 consecutive tiles per XCD (its 8 n-tiles x 4 m-tiles already match
  // about one expert).  Measured at the 16K prefill size; each choice was the
  // faster one for its GEMM.
  const int xcd = blockIdx.x & 7, GX = G >> 3;
  int TS, xcd_base, t_end;
  if (kSwiglu) {
    TS = GX;
    xcd_base = (int)((int64_t)total * xcd / 8) + (blockIdx.x >> 3);
    t_end = (int)((int64_t)total * (xcd + 1) / 8);
  } else {
    TS = G;
    xcd_base = xcd * GX + (blockIdx.x >> 3);
    t_end = total;
  }
  if (xcd_base >= t_end) return;
  const int my_tiles = (t_end - xcd_base + TS - 1) / TS;
  const int wn = wave & 1, wm = wave >> 1;
  const int li = lane & 31, lg = lane >> 5;
  // DMA lane mapping: an instruction fills 8 rows of 128 B; lane l lands at
  // row l/8, physical chunk l%8, which holds logical chunk
  // (l%8) ^ ((row/2)%8); for the 8-row groups at even and odd multiples of 8
  // rows that is (l%8) ^ (l/16) and (l%8) ^ (l/16) ^ 4.
  const int drow = lane >> 3;
  const int dch_even = (lane & 7) ^ (lane >> 4);
  const int dch_odd = dch_even ^ 4;

  auto tile_info = [&](int t) __attribute__((always_inline)) -> TileInfo {
    TileInfo ti;
    const int mt = t / n_tiles;
    ti.nt = t - mt * n_tiles;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tile0[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    ti.e = uni(lo);
    ti.m0 = uni64(s_row0[ti.e] + (int64_t)(mt - s_tile0[ti.e]) * kBM);
    ti.rows_valid = uni((int)std::min<int64_t>(kBM, s_row0[ti.e + 1] - ti.m0));
    return ti;
  };

  // ---- DMA cursor over the stage sequence (tile j, k stage ks) -------------
  // wave w fetches weight rows [32w, 32w+32) (4 x 8 rows) and token rows
  // [kTokRows w, kTokRows (w+1)); waves 0-3 fetch weight scale rows
  // [64w, 64w+64), waves 4.. token scale rows [64(w-4), 64(w-4)+64) (with
  // 128-row tiles waves 6 and 7 fetch no scales).  The cursor never passes the last stage: the
  // fetches issued during the last stage repeat it into the slot no wave
  // reads any more, so every fetch is in bounds and the loop has no branch
  // around its loads.
  struct Src {
    const uint8_t* wrow;   // weight row held in LDS row 32*wave (uniform)
    const uint8_t* arow;   // token row m0 (uniform)
    const uint8_t* srowp;  // scale row base this wave fetches (uniform)
    int last;              // min(M - 1 - m0, kBM - 1): last readable token row of the tile, relative to m0
    int tok;               // nonzero if this wave's kTokRows token rows hold a row of the tile's expert
    int rot;               // the tile's k-stage rotation
  };
  auto make_src = [&](int t) __attribute__((always_inline)) -> Src {
    const TileInfo ti = tile_info(t);
    Src s;
    int64_t wbase, sbase;  // weight rows of this wave's data and scale slabs
    if (kSwiglu) {
      // LDS rows [128h, 128h+64) hold gate rows, [128h+64, 128h+128) up rows
      // of h columns [hc0 + 64h, hc0 + 64h + 64), h = 0, 1
      const int64_t hc0 = (int64_t)ti.nt * (BN / 2);
      const int q = wave & 3;
      wbase = (q < 2 ? 0 : p.I - 64) + hc0 + 64 * (wave >> 2) + 32 * q;
      sbase = ((wave & 1) ? p.I : 0) + hc0 + 64 * ((wave & 3) >> 1);
    } else {
      wbase = (int64_t)ti.nt * BN + 32 * wave;
      sbase = (int64_t)ti.nt * BN + 64 * (wave & 3);
    }
    const int64_t wr = (int64_t)ti.e * p.Nw;
    if constexpr (kPk)   // the tile's first 32 KB stage block
      s.wrow = uniptr(p.w + ((int64_t)ti.e * n_tiles + ti.nt) * (int64_t)nk * (BN * SK));
    else
      s.wrow = uniptr(p.w + (wr + wbase) * (kW4 ? Kd / 2 : Kd));
    s.arow = uniptr(p.a + ti.m0 * Kd);
    s.srowp = wave < 4 ? uniptr(p.ws + (wr + sbase) * srow) : uniptr(p.as + ti.m0 * srow);
    s.last = uni((int)std::min<int64_t>(p.M - 1 - ti.m0, kBM - 1));
    s.tok = kTokRows * wave < ti.rows_valid;
    // GEMM2: tile (expert e, m-tile mt of e, n-tile nt) runs its k stages in
    // the order (nt + mt) % nk, (nt + mt + 1) % nk, ...: tiles that share
    // weight rows (same nt) or token rows (same mt) reach each 128-byte k
    // slice at different times, so one of them takes the L2 miss and the
    // others hit (measured: GEMM2 17 % faster at the 16K prefill size).
    // GEMM1 (16 stages at K = 2048) runs them in plain order: measured 2 %
    // faster than the rotation at that size (the tiles of an XCD that share
    // an operand then fetch each k slice at about the same time, while it is
    // still in L2).  With scale groups (kG = 4) the groups of 4 stages are
    // visited in an order rotated by rot/4 and the stages inside each group
    // rotated by rot%4, so every group is still fetched whole at its first
    // stage.  The accumulation order changes with it, deterministically per
    // tile.
    s.rot = kSwiglu ? 0 : uni((int)((ti.nt + (ti.m0 - s_row0[ti.e]) / kBM) % nk));
    return s;
  };
  // per-lane parts of the DMA offsets
  const uint32_t lane_off_even = (uint32_t)(drow * Kd + dch_even * 16);
  // e2m1 weights: 64-byte row pieces, an instruction fills 16 rows; lane l at
  // row l/4, physical chunk l%4 = logical chunk (l%4) ^ ((row/4)%4)
  const uint32_t lane_off_a4 = (uint32_t)((lane >> 2) * (Kd / 2) + ((((lane & 3) ^ ((lane >> 4) & 3))) << 4));
  const uint32_t lane_off_odd = (uint32_t)(drow * Kd + dch_odd * 16);
  const uint32_t lane_s = (uint32_t)(lane * srow);
  // scale fetch: waves 0-3 weight scales (64 rows from srowp), waves 4-7
  // token scales (rows past M repeat the last row).  Offsets are byte
  // offsets clamped with one min against a scalar cap, so the DMA path has
  // no multiply and no branch.
  uint32_t s_lds = 0;   // kG = 1: the wave's 64 scale words in the slot
  if constexpr (kG == 1)
    s_lds = wave < 4 ? (uint32_t)offsetof(Stage, sa) + (uint32_t)(256 * wave)
                     : (uint32_t)offsetof(Stage, sb) + (uint32_t)(256 * (wave - 4));
  const uint32_t s_lane = wave < 4 ? lane_s : (uint32_t)((64 * (wave - 4) + lane) * srow);
  auto s_voff = [&](int last) __attribute__((always_inline)) -> uint32_t {
    const uint32_t cap = wave < 4 ? 0xffffffffu : (uint32_t)(last * srow);
    return std::min(s_lane, cap);
  };
  // token rows of this wave's B part: row kTokRows wave + 8 j + drow, as a byte offset
  const uint32_t b_row0 = (uint32_t)((kTokRows * wave + drow) * Kd);
  // waves that fetch scale words (all but 6 and 7 with 128-row tiles)
  const bool sc_dma = kBM == 256 || wave < 4 + kBM / 64;
  const uint32_t st_base = lds_addr(&st[0]);
  const uint32_t sc_base = lds_addr(&s_sc[0]);
  // memory k stage of tile stage ks for a tile with rotation rot
  const int n_groups = nk / kG;
  auto kmem = [&](int ks, int rot) __attribute__((always_inline)) -> int {
    if constexpr (kG == 1) {
      const int kr = ks + rot;
      return kr >= nk ? kr - nk : kr;
    } else {
      int grp = (ks >> 2) + (rot >> 2);
      grp = grp >= n_groups ? grp - n_groups : grp;
      return 4 * grp + (((ks & 3) + rot) & 3);
    }
  };
  int cur_r = 0;   // rot % 4 of the tile whose fragments are being read
  // ring slot of global stage gs
  auto slot_of = [](int gs) __attribute__((always_inline)) -> int {
    if constexpr (kSl == 2) return gs & 1;
    else return (int)((unsigned)gs % 3u);
  };
  // VMEM instructions this wave issues for the DMA of tile stage ks (kSl =
  // 3: the mid-stage wait leaves the latest stage in flight; loads retire in
  // order, so the count must be exact); with kG = 4 only a group's first
  // stage carries the scale load
  auto dma_count = [&](const Src& src, int ks) __attribute__((always_inline)) -> int {
    return kNA + (src.tok ? kNT : 0) + ((sc_dma && (kG == 1 || (ks & 3) == 0)) ? 1 : 0);
  };
  const uint32_t s_lds4 = wave < 4 ? (uint32_t)(1024 * wave) : (uint32_t)(BN * 16 + 1024 * (wave - 4));
  // One DMA instruction of k stage ks of the tile whose source is `src`,
  // global stage gs (ring slot gs%2): i = 0..3 weight rows, 4..7 token rows,
  // 8 scales.
  auto dma_part = [&](int i, const Src& src, int ks, int gs) __attribute__((always_inline)) {
    const uint32_t base = st_base + (uint32_t)slot_of(gs) * (uint32_t)sizeof(Stage);
    const int kr = kmem(ks, src.rot);   // the k stage in memory
    const uint32_t ko = (uint32_t)(kr * SK);
    // the row and k offsets go into the per-lane 32-bit offset, so the only
    // scalar operand is the row base
    if (i < kNA) {
      if constexpr (kW4) {
        dma16(lane_off_a4 + (uint32_t)(8 * i * Kd) + (uint32_t)(kr * (SK / 2)), src.wrow,
              base + (uint32_t)offsetof(Stage, a) + (uint32_t)((32 * wave + 16 * i) * (SK / 2)));
      } else if constexpr (kPk) {
        // 1 KB contiguous: slot rows 32 wave + 8 i .. + 8, chunks as stored
        dma16((uint32_t)(kr * (BN * SK)) + (uint32_t)((32 * wave + 8 * i) * SK) + (uint32_t)(lane * 16), src.wrow,
              base + (uint32_t)offsetof(Stage, a) + (uint32_t)((32 * wave + 8 * i) * SK));
      } else {
        dma16(((i & 1) ? lane_off_odd : lane_off_even) + (uint32_t)(8 * i * Kd) + ko, src.wrow,
              base + (uint32_t)offsetof(Stage, a) + (uint32_t)((32 * wave + 8 * i) * SK));
      }
    } else if (i < kNA + kNT) {
      const int j = i - kNA;
      // rows past M repeat the last row
      const uint32_t row = std::min(b_row0 + (uint32_t)(8 * j * Kd), (uint32_t)(src.last * Kd));
      const uint32_t voff = row + (uint32_t)(((j & 1) ? dch_odd : dch_even) * 16) + ko;
      // a ragged tail tile skips token rows past its expert's rows: only the
      // outputs of those (never stored) rows read what stays in LDS there
      if (src.tok)
        dma16(voff, src.arow, base + (uint32_t)offsetof(Stage, b) + (uint32_t)((kTokRows * wave + 8 * j) * SK));
    } else if constexpr (kG == 1) {
      if (sc_dma) dma4(s_voff(src.last) + (uint32_t)(kr * 4), src.srowp, base + s_lds);
    } else if (sc_dma && (ks & 3) == 0) {
      // the group's 16 bytes per row, from its first stage in memory (with
      // 128-row tiles waves 6 and 7 have no scale rows: their ring offsets
      // would lie past the 6 KB group buffer)
      dma16(s_voff(src.last) + (uint32_t)((kr & ~3) * 4), src.srowp,
            sc_base + (uint32_t)(((gs >> 2) & 1) * kScBuf) + s_lds4);
    }
  };
  auto dma_stage = [&](const Src& src, int ks, int gs) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kDmaOps; ++i) dma_part(i, src, ks, gs);
  };

  // ---- LDS read addresses: row (li) part and the swizzled chunk parts ------
  // Fragment rows differ by multiples of 32, so (row/2)%8 = (li/2)%8 for all.
  const int sw = (li >> 1) & 7;
  const uint32_t rd_a = (uint32_t)offsetof(Stage, a) + (uint32_t)((128 * wn + li) * kRowA);
  const uint32_t rd_b = (uint32_t)offsetof(Stage, b) + (uint32_t)((32 * kNB * wm + li) * SK);
  uint32_t rd_sa = 0, rd_sb = 0;   // kG = 1: scale words in the slot
  if constexpr (kG == 1) {
    rd_sa = (uint32_t)offsetof(Stage, sa) + (uint32_t)((128 * wn + li) * 4);
    rd_sb = (uint32_t)offsetof(Stage, sb) + (uint32_t)((32 * kNB * wm + li) * 4);
  }
  const uint32_t rd_sa4 = (uint32_t)((128 * wn + li) * 16);          // kG = 4 scale ring
  const uint32_t rd_sb4 = (uint32_t)(BN * 16 + (32 * kNB * wm + li) * 16);
  uint32_t chk[4];   // byte offset of logical chunk 2c + lg within a row
#pragma unroll
  for (int c = 0; c < 4; ++c) chk[c] = (uint32_t)(((2 * c + lg) ^ sw) << 4);
  // Fragments of one 64-wide k sub-step: A rows 128 wn + 32 f + li, B rows
  // 64 wm + 32 f + li; sub-step s covers logical chunks {4s + lg, 4s + 2 + lg}
  // of a row and scale byte 2s + lg of its stage word (read as one byte, so
  // the value goes to the MFMA with no arithmetic between load and use).
  auto slot_ptr = [&](int slot) __attribute__((always_inline)) {
    uint32_t b = st_base + (uint32_t)slot * (uint32_t)sizeof(Stage);
    asm("" : "+s"(b));   // opaque: one add per load instead of both slots' addresses kept live
    return (const lds_u8*)(uintptr_t)b;
  };
  // e2m1 fragment of sub-step s: lane group g holds the 32 codes of k block
  // g (k [64s + 32g, +32)), i.e. bytes [32s + 16g, +16) of the row's piece:
  // logical chunk 2s + lg, stored at (2s + lg) ^ ((row/4)%4); (row/4)%4 =
  // (li/4)%4 for every fragment row
  uint32_t chk4[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) chk4[c] = (uint32_t)(((2 * c + lg) ^ ((li >> 2) & 3)) << 4);
  // kG = 4: the scale bytes of global stage gs (tile stage ks = gs mod nk,
  // tiles start at multiples of 4) sit at word (ks + rot) % 4 of each row's
  // 16 bytes in group buffer (gs/4)%2
  auto group_ptr = [&](int gs) __attribute__((always_inline)) {
    uint32_t b = sc_base + (uint32_t)(((gs >> 2) & 1) * kScBuf + (((gs & 3) + cur_r) & 3) * 4);
    asm("" : "+s"(b));
    return (const lds_u8*)(uintptr_t)b;
  };
  // fragments of global stage gs (ring slot gs%2)
  auto load_a = [&](int gs, int s, int f, v8i& frag, int& sc) __attribute__((always_inline)) {
    const lds_u8* S = slot_ptr(slot_of(gs));
    const lds_u8* pa = S + rd_a + f * 32 * kRowA;
    if constexpr (kW4) {
      const u32x4 a0 = *reinterpret_cast<lds_u32x4_v*>(pa + chk4[s]);
      frag = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
    } else {
      const u32x4 a0 = *reinterpret_cast<lds_u32x4_v*>(pa + chk[2 * s]);
      const u32x4 a1 = *reinterpret_cast<lds_u32x4_v*>(pa + chk[2 * s + 1]);
      frag = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
    if constexpr (kG == 1)
      sc = (int)*reinterpret_cast<lds_u8_v*>(S + rd_sa + f * 128 + 2 * s + lg);
    else
      sc = (int)*reinterpret_cast<lds_u8_v*>(group_ptr(gs) + rd_sa4 + f * 512 + 2 * s + lg);
  };
  auto load_b = [&](int gs, int s, int f, v8i& frag, int& sc) __attribute__((always_inline)) {
    const lds_u8* S = slot_ptr(slot_of(gs));
    const lds_u8* pb = S + rd_b + f * 32 * SK;
    const u32x4 b0 = *reinterpret_cast<lds_u32x4_v*>(pb + chk[2 * s]);
    const u32x4 b1 = *reinterpret_cast<lds_u32x4_v*>(pb + chk[2 * s + 1]);
    frag = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    if constexpr (kG == 1)
      sc = (int)*reinterpret_cast<lds_u8_v*>(S + rd_sb + f * 128 + 2 * s + lg);
    else
      sc = (int)*reinterpret_cast<lds_u8_v*>(group_ptr(gs) + rd_sb4 + f * 512 + 2 * s + lg);
  };
  // ---- schedule ---------------------------------------------------------------
  // Stage g (tile-local k stage ks) lives in slot g%S (S = kSl slots).
  // Sub-step 0 of stage g runs on fragments loaded during the previous
  // sub-step and reloads them for sub-step 1 from the same slot.  Then one
  // barrier: every wave is done reading slot g%S and (after its own vmcnt
  // wait) every part of stage g+1 has landed.  Sub-step 1 reloads the
  // fragments of stage g+1's sub-step 0 and, after its first two MFMAs,
  // issues the DMA of stage g+S into slot g%S, S-1 stages ahead of its use
  // (with S = 3 the wait leaves that latest DMA in flight).  A tile's last
  // stage issues no DMA: its slot holds the epilogue's staging, and the DMA
  // that was skipped follows the epilogue.

  // prologue: stages 0 .. S-1 in flight
  const Src first = make_src(xcd_base);
  if constexpr (kSl == 3) {   // nk >= 3 (host)
    dma_stage(first, 0, 0);
    dma_stage(first, 1, 1);
    dma_stage(first, 2, 2);
  } else if (nk > 1) {
    dma_stage(first, 0, 0);
    dma_stage(first, 1, 1);
  } else {
    dma_stage(first, 0, 0);
    if (my_tiles > 1) dma_stage(make_src(TS + xcd_base), 0, 1);
  }
  wait_vmcnt0();
  barrier();

  int g = 0;          // global stage index
  int last_cnt = 0;   // kSl = 3: VMEM instructions of this wave's latest stage DMA
  for (int cj = 0; cj < my_tiles; ++cj) {
    const TileInfo cur = tile_info(cj * TS + xcd_base);
    // Ragged tail tiles: a wave whose 32 kNB tokens are all past the
    // expert's rows computes nothing (no fragment loads, MFMAs or epilogue
    // work); it still issues its share of the weight DMA and meets every
    // barrier.
    const bool active = 32 * kNB * wm < cur.rows_valid;
    const Src csrc = make_src(cj * TS + xcd_base);
    cur_r = csrc.rot & 3;
    const bool has_next = cj + 1 < my_tiles;
    const Src nsrc = has_next ? make_src((cj + 1) * TS + xcd_base) : csrc;
    v8i fa[4], fb[kNB];
    int sa[4], sb[kNB];
    v16f acc[4][kNB];
    // The 4 kNB MFMAs of one sub-step, B fragment 0 with A fragments 0..3,
    // then B fragment 1 with A 0..3.  Each fragment is reloaded for the next
    // sub-step (stage `nstage`, sub-step `ns`) right after its last MFMA, so
    // the LDS reads overlap the matrix work; `extra(m)` runs after MFMA m
    // (DMA issue).
    auto substep = [&](int nstage, int ns, auto kReload, auto extra) __attribute__((always_inline)) {
      if (!active) {
  #pragma unroll
        for (int m = 0; m < 4 * kNB; ++m) extra(m);
        return;
      }
  #pragma unroll
      for (int m = 0; m < 4 * kNB; ++m) {
        const int fm = m >> 2, fn = m & 3;
        // A format 4 = e2m1 (W4A8), 0 = e4m3; B (tokens) is always e4m3
        acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[fn], fb[fm], acc[fn][fm], kW4 ? 4 : 0, 0, 0,
                                                                       sa[fn], 0, sb[fm]);
        // pin the MFMA here: without a use at this point the optimiser sinks
        // the (side-effect free) MFMAs below the loads that were meant to
        // overlap them, which also lengthens every fragment's live range
        asm volatile("" : "+v"(acc[fn][fm]));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(kReload)::value) {
          if constexpr (kNB == 2) {
            if (m == 3) load_b(nstage, ns, 0, fb[0], sb[0]);
            if (m >= 4) load_a(nstage, ns, m - 4, fa[m - 4], sa[m - 4]);
            if (m == 7) load_b(nstage, ns, 1, fb[1], sb[1]);
          } else {
            load_a(nstage, ns, m, fa[m], sa[m]);
            if (m == 3) load_b(nstage, ns, 0, fb[0], sb[0]);
          }
        }
        extra(m);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto load_all = [&](int gs, int s) __attribute__((always_inline)) {
  #pragma unroll
      for (int f = 0; f < 4; ++f) load_a(gs, s, f, fa[f], sa[f]);
  #pragma unroll
      for (int f = 0; f < kNB; ++f) load_b(gs, s, f, fb[f], sb[f]);
    };
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < kNB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;
    // the tile's first fragments (stage g has landed: the prologue's barrier,
    // or the middle barrier of the previous tile's last stage)
    if (active) load_all(g, 0);

    // one k stage; kDma: issue stage g+S's DMA (every stage but the tile's last)
    auto stage = [&](int ks, auto kDma) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      substep(g, 1, std::true_type{}, [&](int) {});
      // this wave's part of stage g+1 has landed (S = 3: stage g+2's DMA,
      // the latest, may still be in flight)
      if constexpr (kSl == 2) wait_vmcnt0(); else wait_vmcnt_le(last_cnt);
      barrier();       // every wave's has, and nobody reads slot g%S any more
      if constexpr (decltype(kDma)::value) {
        // DMA target: stage ks+S of this tile, else stage ks+S-nk of the next
        // tile, else (last tile) a repeat of this tile's last stage, never read
        const bool in_tile = ks + kSl < nk;
        Src t;
        t.wrow = in_tile ? csrc.wrow : nsrc.wrow;
        t.arow = in_tile ? csrc.arow : nsrc.arow;
        t.srowp = in_tile ? csrc.srowp : nsrc.srowp;
        t.last = in_tile ? csrc.last : nsrc.last;
        t.tok = in_tile ? csrc.tok : nsrc.tok;
        t.rot = in_tile ? csrc.rot : nsrc.rot;
        // (S = 2: only stage nk-2 reaches past the tile, to the next tile's stage 0)
        const int tks = in_tile ? ks + kSl : (has_next ? (kSl == 2 ? 0 : ks + kSl - nk) : nk - 1);
        // the DMA goes out early in the sub-step (measured: issuing it over
        // all eight MFMAs leaves the last loads too little time to land)
        substep(g + 1, 0, std::true_type{}, [&](int m) __attribute__((always_inline)) {
          if (m == 0) {
#pragma unroll
            for (int i = 0; i < 5; ++i) dma_part(i, t, tks, g + kSl);
          }
          if (m == 1) {
#pragma unroll
            for (int i = 5; i < kDmaOps; ++i) dma_part(i, t, tks, g + kSl);
          }
        });
        if constexpr (kSl == 3) last_cnt = dma_count(t, tks);
      } else {
        substep(g + 1, 0, std::false_type{}, [&](int) {});   // the next tile reloads at its start
      }
      __builtin_amdgcn_sched_barrier(0);
      ++g;
    };
    for (int ks = 0; ks + 1 < nk; ++ks) stage(ks, std::true_type{});
    stage(nk - 1, std::false_type{});

    // ---- epilogue (the next tile's first stage has landed) -------------------
    if (!kSwiglu) {
      // The bf16 tile goes out through LDS so that every store writes whole
      // 128-byte lines: each wave stages its 32-token x 128-feature halves
      // (8 KB each) in its own part of the ring slot the last stage was read
      // from (no wave reads it and no DMA targets it any more), then reads
      // them back row-contiguous.  Staging layout: token row r at r*256;
      // 16-byte chunk c at physical chunk c ^ (r%16), and its two 8-byte
      // halves swapped when r >= 16, so both the writes (lane = token) and
      // the reads (16 lanes per row) are free of bank conflicts.  With
      // 128-row tiles the 8 KB per wave do not fit one 48 KB slot for all 8
      // waves: waves 0-3 go first, then (after a barrier) waves 4-7 reuse the
      // same regions.
      const int64_t N = p.Nw;
      constexpr int kRounds = kBM == 256 ? 1 : 2;
#pragma unroll
      for (int round = 0; round < kRounds; ++round) {
      if (kRounds == 2 && round == 1) barrier();   // round 0's read-backs are done
      if (active && (kRounds == 1 || (wave >> 2) == round)) {
      const int li = opaque(lane & 31), lg = opaque(lane >> 5), lane_e = opaque(lane);
      lds_u8* stg = (lds_u8*)(uintptr_t)(st_base + (uint32_t)slot_of(g - 1) * (uint32_t)sizeof(Stage) +
                                         (uint32_t)((kRounds == 1 ? wave : (wave & 3)) * 8192));
      const int rr = lane_e >> 4, rc = lane_e & 15;   // read-back: row within a group of 4, chunk
#pragma unroll
      for (int fm = 0; fm < kNB; ++fm) {
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v16f& c = acc[fn][fm];
            const u32x2 o = {pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3])};
            const int chunk = (4 * fn + q) ^ (li & 15);
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                stg + li * 256 + chunk * 16 + ((lg ^ (li >> 4)) << 3)) = o;
          }
        asm volatile("" ::: "memory");   // a wave's LDS accesses execute in issue order
        u32x4 v[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int r = 4 * it + rr;
          v[it] = *reinterpret_cast<lds_u32x4*>(stg + r * 256 + ((rc ^ (r & 15)) << 4));
          if (it >= 4) v[it] = u32x4{v[it].z, v[it].w, v[it].x, v[it].y};   // rows 16-31
        }
        const int mc0 = 32 * kNB * wm + 32 * fm + rr;
        uint16_t* y0 = p.y + (cur.m0 + mc0) * N + (int64_t)cur.nt * BN + 128 * wn + 8 * rc;
#pragma unroll
        for (int it = 0; it < 8; ++it)
          if (mc0 + 4 * it < cur.rows_valid)
            __builtin_nontemporal_store(v[it], reinterpret_cast<u32x4*>(y0 + 4 * it * N));
        asm volatile("" ::: "memory");   // a wave's LDS accesses execute in issue order
      }
      }   // active
      }   // round
    } else {
      // SwiGLU, MX requant, and the stores through LDS: the two waves that
      // share a block of kTB = 32 kNB tokens (wn = 0, 1: 64 h columns each)
      // stage their e4m3 bytes into one kTB x 128-byte region (16-byte chunk
      // index XOR-ed with (row/2)%8) and their scale bytes into kTB x 4
      // bytes, so after a barrier every row of the tile leaves as one full
      // 128-byte line and one 4-byte scale word.
      constexpr int kTB = 32 * kNB;
      const int64_t I = p.I;
      const int li = opaque(lane & 31), lg = opaque(lane >> 5), lane_e = opaque(lane);
      lds_u8* grp = (lds_u8*)(uintptr_t)(st_base + (uint32_t)slot_of(g - 1) * (uint32_t)sizeof(Stage) +
                                         (uint32_t)(wm * (kTB * 128 + kTB * 4)));
      lds_u8* grp_s = grp + kTB * 128;
      // (both waves of a group are active or neither: they share wm)
#pragma unroll
      for (int fm = 0; fm < kNB; ++fm) {
        if (!active) break;
        const int t = 32 * fm + li;   // token row within the kTB-token block
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          __builtin_amdgcn_sched_barrier(0);   // one 32x32 block at a time
          // gate fragment f pairs with up fragment f + 2 (same h columns)
          float h[16];
          float amax = 0.0f;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            h[v] = swiglu(acc[f][fm][v], acc[f + 2][fm][v]);
            amax = fmaxf(amax, fabsf(h[v]));
          }
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const uint32_t sbyte = e8m0_from_amax(amax);
          const float inv = e8m0_inverse(sbyte);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int hc = 64 * wn + 32 * f + 8 * q + 4 * lg;   // h column within the tile
            const int phys = ((hc >> 4) ^ ((t >> 1) & 7)) << 4 | (hc & 15);
            *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(grp + t * 128 + phys) =
                e4m3x4(h[4 * q] * inv, h[4 * q + 1] * inv, h[4 * q + 2] * inv, h[4 * q + 3] * inv);
          }
          if (lg == 0) grp_s[t * 4 + 2 * wn + f] = static_cast<uint8_t>(sbyte);
          if (p.hdbg && kTB * wm + t < cur.rows_valid) {
            float* drow_ = p.hdbg + (cur.m0 + kTB * wm + t) * I + (int64_t)cur.nt * (BN / 2) + 64 * wn + 32 * f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(drow_ + 8 * q + 4 * lg) =
                  make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
          }
        }
      }
      barrier();
      // wave wn stores rows [kTB/2 wn, kTB/2 (wn + 1)) of its group: 8 lanes per row
      if (active) {
      constexpr int kHR = kTB / 2;   // rows per wave
      const int64_t hc0 = (int64_t)cur.nt * (BN / 2);
      u32x4 v[kHR / 8];
#pragma unroll
      for (int it = 0; it < kHR / 8; ++it) {
        const int r = kHR * wn + 8 * it + (lane_e >> 3);
        v[it] = *reinterpret_cast<lds_u32x4*>(grp + r * 128 + ((((lane_e & 7) ^ ((r >> 1) & 7))) << 4));
      }
      const uint32_t sw_word = li < kHR ? *reinterpret_cast<lds_u32*>(grp_s + (kHR * wn + li) * 4) : 0u;
#pragma unroll
      for (int it = 0; it < kHR / 8; ++it) {
        const int r = kHR * wn + 8 * it + (lane_e >> 3);
        if (kTB * wm + r < cur.rows_valid)
          *reinterpret_cast<u32x4*>(p.hq + (cur.m0 + kTB * wm + r) * I + hc0 + 16 * (lane_e & 7)) = v[it];
      }
      if (lg == 0 && (kHR == 32 || li < kHR) && kTB * wm + kHR * wn + li < cur.rows_valid)
        *reinterpret_cast<uint32_t*>(p.hs + (cur.m0 + kTB * wm + kHR * wn + li) * (I / 32) + hc0 / 32) = sw_word;
      }   // active
    }
    // every wave is done with the staging slot: issue the DMA the last stage
    // skipped, global stage g + S - 1 (the next tile's stage S - 1, or with
    // one stage per tile the stage 0 of the tile after next)
    barrier();
    if constexpr (kSl == 3) {
      if (has_next) {
        dma_stage(nsrc, 2, g + 2);
        last_cnt = dma_count(nsrc, 2);
      }
    } else if (nk > 1) {
      if (has_next) dma_stage(nsrc, 1, g + 1);
    } else if (cj + 2 < my_tiles) {
      dma_stage(make_src((cj + 2) * TS + xcd_base), 0, g + 1);
    }
  }
  // outstanding DMA must land before the workgroup's LDS is released
  wait_vmcnt0();
}

// 128-row tiles (three-slot ring) when the experts average at most this
// many rows, where a 256-row tile is at most a quarter full and the GEMMs
// stream weights rather than compute.  Measured on the layer: decode
// (2 rows per expert) 157 -> 138 us; at 128 rows per expert (T = 2048,
// top-8 of 128) the 128-row tiles were 2 % slower.
constexpr int64_t kSmallRowsPerExpert = 64;

template <bool kSwiglu, int kWF>
int launch(const GmmParams& p, hipStream_t stream, const char* name) {
  if (p.M == 0) return MX_OK;
  const bool small = p.Kd / BK >= 3 && p.gl_type != kGlSingle && p.M <= kSmallRowsPerExpert * p.E;
  const int64_t bm = small ? 128 : BM;
  const int64_t upper = ((p.M + bm - 1) / bm + p.E) * (int64_t)p.n_tiles;
  if (upper >= ((int64_t)1 << 31)) return fail(MX_ERR_UNSUPPORTED, "%s: too many tiles", name);
  int64_t grid = (int64_t)num_cus() / 8 * 8;
  if (grid < 8) grid = 8;
  if (grid > (upper + 7) / 8 * 8) grid = (upper + 7) / 8 * 8;
  const dim3 g3((unsigned)grid), b3(kThreads);
  // the per-expert tables (dynamic LDS)
  const size_t tab = (size_t)(p.E + 1) * 2 * sizeof(int);
  // scale groups of 4 stages when the k stages divide into them and both
  // scale tensors are 16-byte aligned (every scale row then is); with
  // 128-row tiles also only while the scale ring fits beside the three slots
  const bool groups = (p.Kd / BK) % 4 == 0 && reinterpret_cast<uintptr_t>(p.as) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(p.ws) % 16 == 0;
  if (small) {
    // LDS left for the tables beside that kernel's static LDS (as compiled),
    // read once; 0 if the query fails (then per-stage scale loads)
    static const size_t room = [] {
      hipFuncAttributes a{};
      int dev = 0, lim = 0;
      if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(gmm_kernel<kSwiglu, kWF, 4, 128>)) != hipSuccess ||
          hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
        (void)hipGetLastError();
        return (size_t)0;
      }
      return a.sharedSizeBytes < (size_t)lim ? (size_t)lim - a.sharedSizeBytes : (size_t)0;
    }();
    if (groups && tab <= room)
      gmm_kernel<kSwiglu, kWF, 4, 128><<<g3, b3, tab, stream>>>(p);
    else
      gmm_kernel<kSwiglu, kWF, 1, 128><<<g3, b3, tab, stream>>>(p);
    return check_launch(name);
  }
  if (groups)
    gmm_kernel<kSwiglu, kWF, 4, 256><<<g3, b3, tab, stream>>>(p);
  else
    gmm_kernel<kSwiglu, kWF, 1, 256><<<g3, b3, tab, stream>>>(p);
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
  // the DMA addresses a tile's 256 rows with 32-bit byte offsets
  if (Kd > kMaxKd) return fail(MX_ERR_UNSUPPORTED, "%s: reduction size %lld > %lld", name, (long long)Kd,
                               (long long)kMaxKd);
  if (E > kMaxE) return fail(MX_ERR_UNSUPPORTED, "%s: E=%lld > %d", name, (long long)E, kMaxE);
  if (M >= (int64_t)1 << 31) return fail(MX_ERR_UNSUPPORTED, "%s: M >= 2^31", name);
  return MX_OK;
}

int launch_gmm_mx(const uint8_t* a, const uint8_t* as, const uint8_t* w, const uint8_t* ws,
                  const int64_t* gl, int gl_type, int64_t M, int64_t N, int64_t Kd, int64_t E, uint16_t* y,
                  hipStream_t stream, int wf) {
  GmmParams p{};
  p.a = a; p.as = as; p.w = w; p.ws = ws; p.group_list = gl; p.gl_type = gl_type;
  p.E = (int)E; p.M = M; p.Kd = Kd; p.Nw = N; p.n_tiles = (int)(N / BN); p.y = y;
  if (wf == kWfE2m1) return launch<false, kWfE2m1>(p, stream, "gmm_mx_w4a8");
  if (wf == kWfPacked) return launch<false, kWfPacked>(p, stream, "gmm_mx_packed");
  return launch<false, kWfE4m3>(p, stream, "gmm_mx");
}

int launch_gmm_swiglu(const uint8_t* a, const uint8_t* as, const uint8_t* w13, const uint8_t* w13s,
                      const int64_t* gl, int gl_type, int64_t M, int64_t K, int64_t I, int64_t E, uint8_t* hq,
                      uint8_t* hs, float* hdbg, hipStream_t stream, int wf) {
  GmmParams p{};
  p.a = a; p.as = as; p.w = w13; p.ws = w13s; p.group_list = gl; p.gl_type = gl_type;
  p.E = (int)E; p.M = M; p.Kd = K; p.Nw = 2 * I; p.n_tiles = (int)(I / (BN / 2)); p.I = I;
  p.hq = hq; p.hs = hs; p.hdbg = hdbg;
  if (wf == kWfE2m1) return launch<true, kWfE2m1>(p, stream, "gmm_swiglu_mxquant_w4a8");
  if (wf == kWfPacked) return launch<true, kWfPacked>(p, stream, "gmm_swiglu_mxquant_packed");
  return launch<true, kWfE4m3>(p, stream, "gmm_swiglu_mxquant");
}

}  // namespace mxmoe

namespace {

// Host checks shared by the e4m3 and e2m1 (W4A8) entry points of GEMM2.
int gmm_mx_entry(const char* name, int wf, const void* a_u8, const void* a_s, const void* w_u8, const void* w_s,
                 const int64_t* group_list, int group_list_type, int64_t M, int64_t N, int64_t Kd, int64_t E,
                 void* y_bf16, void* stream) {
  using namespace mxmoe;
  int rc = check_gmm_common(name, group_list_type, M, Kd, E);
  if (rc) return rc;
  if (N <= 0) return fail(MX_ERR_INVALID_ARG, "%s: bad N=%lld", name, (long long)N);
  if (!dims_in_range({N})) return fail(MX_ERR_UNSUPPORTED, "%s: N above 2^31 - 1", name);
  if (N % BN != 0) return fail(MX_ERR_UNSUPPORTED, "%s: N=%lld is not a multiple of %d", name, (long long)N, BN);
  if (!group_list || (M > 0 && (!a_u8 || !a_s || !w_u8 || !w_s || !y_bf16)))
    return fail(MX_ERR_INVALID_ARG, "%s: null pointer", name);
  if (reinterpret_cast<uintptr_t>(a_u8) % 16 || reinterpret_cast<uintptr_t>(w_u8) % 16 ||
      reinterpret_cast<uintptr_t>(a_s) % 4 || reinterpret_cast<uintptr_t>(w_s) % 4 ||
      reinterpret_cast<uintptr_t>(y_bf16) % 16)
    return fail(MX_ERR_UNSUPPORTED, "%s: misaligned pointer", name);
  return launch_gmm_mx(static_cast<const uint8_t*>(a_u8), static_cast<const uint8_t*>(a_s),
                       static_cast<const uint8_t*>(w_u8), static_cast<const uint8_t*>(w_s), group_list,
                       group_list_type, M, N, Kd, E, static_cast<uint16_t*>(y_bf16), as_stream(stream), wf);
}

// Host checks shared by the e4m3 and e2m1 (W4A8) entry points of GEMM1.
int gmm_swiglu_entry(const char* name, int wf, const void* a_u8, const void* a_s, const void* w13_u8,
                     const void* w13_s, const int64_t* group_list, int group_list_type, int64_t M, int64_t K,
                     int64_t I, int64_t E, void* hq_u8, void* hs_u8, float* h_f32_debug, void* stream) {
  using namespace mxmoe;
  int rc = check_gmm_common(name, group_list_type, M, K, E);
  if (rc) return rc;
  if (I <= 0) return fail(MX_ERR_INVALID_ARG, "%s: bad I=%lld", name, (long long)I);
  if (!dims_in_range({I})) return fail(MX_ERR_UNSUPPORTED, "%s: I above 2^31 - 1", name);
  if (I % (BN / 2) != 0)
    return fail(MX_ERR_UNSUPPORTED, "%s: I=%lld is not a multiple of %d", name, (long long)I, BN / 2);
  if (!group_list || (M > 0 && (!a_u8 || !a_s || !w13_u8 || !w13_s || !hq_u8 || !hs_u8)))
    return fail(MX_ERR_INVALID_ARG, "%s: null pointer", name);
  if (reinterpret_cast<uintptr_t>(a_u8) % 16 || reinterpret_cast<uintptr_t>(w13_u8) % 16 ||
      reinterpret_cast<uintptr_t>(a_s) % 4 || reinterpret_cast<uintptr_t>(w13_s) % 4 ||
      reinterpret_cast<uintptr_t>(hq_u8) % 16 || reinterpret_cast<uintptr_t>(hs_u8) % 4 ||
      reinterpret_cast<uintptr_t>(h_f32_debug) % 16)
    return fail(MX_ERR_UNSUPPORTED, "%s: misaligned pointer", name);
  return launch_gmm_swiglu(static_cast<const uint8_t*>(a_u8), static_cast<const uint8_t*>(a_s),
                           static_cast<const uint8_t*>(w13_u8), static_cast<const uint8_t*>(w13_s), group_list,
                           group_list_type, M, K, I, E, static_cast<uint8_t*>(hq_u8),
                           static_cast<uint8_t*>(hs_u8), h_f32_debug, as_stream(stream), wf);
}

}  // namespace

extern "C" int gmm_mx(const void* a_u8, const void* a_s, const void* w_u8, const void* w_s,
                      const int64_t* group_list, int group_list_type, int64_t M, int64_t N, int64_t Kd,
                      int64_t E, void* y_bf16, void* stream) {
  return gmm_mx_entry("gmm_mx", mxmoe::kWfE4m3, a_u8, a_s, w_u8, w_s, group_list, group_list_type, M, N, Kd, E, y_bf16,
                      stream);
}

extern "C" int gmm_mx_w4a8(const void* a_u8, const void* a_s, const void* w_u8, const void* w_s,
                           const int64_t* group_list, int group_list_type, int64_t M, int64_t N, int64_t Kd,
                           int64_t E, void* y_bf16, void* stream) {
  return gmm_mx_entry("gmm_mx_w4a8", mxmoe::kWfE2m1, a_u8, a_s, w_u8, w_s, group_list, group_list_type, M, N, Kd, E,
                      y_bf16, stream);
}

extern "C" int gmm_swiglu_mxquant(const void* a_u8, const void* a_s, const void* w13_u8, const void* w13_s,
                                  const int64_t* group_list, int group_list_type, int64_t M, int64_t K,
                                  int64_t I, int64_t E, void* hq_u8, void* hs_u8, float* h_f32_debug,
                                  void* stream) {
  return gmm_swiglu_entry("gmm_swiglu_mxquant", mxmoe::kWfE4m3, a_u8, a_s, w13_u8, w13_s, group_list, group_list_type, M,
                          K, I, E, hq_u8, hs_u8, h_f32_debug, stream);
}

extern "C" int gmm_swiglu_mxquant_w4a8(const void* a_u8, const void* a_s, const void* w13_u8, const void* w13_s,
                                       const int64_t* group_list, int group_list_type, int64_t M, int64_t K,
                                       int64_t I, int64_t E, void* hq_u8, void* hs_u8, float* h_f32_debug,
                                       void* stream) {
  return gmm_swiglu_entry("gmm_swiglu_mxquant_w4a8", mxmoe::kWfE2m1, a_u8, a_s, w13_u8, w13_s, group_list,
                          group_list_type, M, K, I, E, hq_u8, hs_u8, h_f32_debug, stream);
}

extern "C" int gmm_mx_packed(const void* a_u8, const void* a_s, const void* w_packed, const void* w_s,
                             const int64_t* group_list, int group_list_type, int64_t M, int64_t N, int64_t Kd,
                             int64_t E, void* y_bf16, void* stream) {
  return gmm_mx_entry("gmm_mx_packed", mxmoe::kWfPacked, a_u8, a_s, w_packed, w_s, group_list, group_list_type, M,
                      N, Kd, E, y_bf16, stream);
}

extern "C" int gmm_swiglu_mxquant_packed(const void* a_u8, const void* a_s, const void* w13_packed,
                                         const void* w13_s, const int64_t* group_list, int group_list_type,
                                         int64_t M, int64_t K, int64_t I, int64_t E, void* hq_u8, void* hs_u8,
                                         float* h_f32_debug, void* stream) {
  return gmm_swiglu_entry("gmm_swiglu_mxquant_packed", mxmoe::kWfPacked, a_u8, a_s, w13_packed, w13_s, group_list,
                          group_list_type, M, K, I, E, hq_u8, hs_u8, h_f32_debug, stream);
}
