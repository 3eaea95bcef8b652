// Large-tile NT GEMM on MFMA 32x32x16: C[M, N] = A[M, K] . B[N, K]^T with
// bf16 operands (both K-contiguous), fp32 accumulation, bf16 or fp32 output.
// Used for the many-token (prefill) decomposed linear: both stages, x U_r and
// t V_r, have this form with the factors stored transposed.
//
// Tile 256 x BN x BK (BN = 256 or 128), one workgroup of 8 waves, each wave
// 64 x BN/2.  Operand tiles move global -> LDS with direct-to-LDS buffer
// loads (no registers in between) through a ring of NS stages: the loads of
// the next NS - 1 k-tiles are in flight while one multiplies.  LDS rows are
// BK * 2 bytes with the 16-byte chunk index XOR-swizzled by row, so the
// fragment reads (32 rows at one chunk) spread over the banks.  The MFMA
// takes the B fragment as its first operand, so each lane ends with 4
// consecutive output columns of one row; bf16 results are staged through LDS
// and written as whole 128-byte lines, with non-temporal stores (the output
// is not read again by this launch, and streaming it past the L2 leaves the
// operands' lines there).  Tiles are listed four row tiles at a
// time and go to the 8 XCDs in contiguous runs of that list (workgroups are
// dealt to XCDs round robin), so the tiles an XCD runs at once share A and B
// rows in its L2.  Rows past M or N and k-chunks past K read zero from
// outside the buffers; the padding in the last partial chunk is zeroed in
// LDS.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int gBM = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 16-byte chunk slot of (row, chunk) in a staged tile with BK * 2-byte rows:
// 16 consecutive rows at one chunk land in 16 distinct slots of a 256-byte
// bank window.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  return BK == 64 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}

template <int VM>
__device__ __forceinline__ void wait_vm() {
  // vmcnt(VM); expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS loads of a ROWS x BK operand tile: instruction i moves the
// 1 KB of rows RPI*i .. RPI*i + RPI-1 (lane l: row RPI*i + l/CPR, LDS slot
// l%CPR, global chunk swizzled), and wave w of NW issues instructions w,
// w + NW, ...; chunks past the K range (kt elements left) go outside the
// buffer and read zero.
template <int ROWS, int BK, int NW>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int kt,
                                          uint8_t* lds, int wave, int lane) {
  constexpr int CPR = BK / 8, RPI = 64 / CPR;
  static_assert(ROWS % (RPI * NW) == 0, "whole instructions per wave");
  const int rr = lane / CPR, slot = lane % CPR;
#pragma unroll
  for (int i = 0; i < ROWS / RPI / NW; ++i) {
    const int inst = wave + NW * i;
    const int row = inst * RPI + rr;
    const int chunk = swz<BK>(row, slot);
    const int off =
        chunk * 8 < kt ? (int)(((int64_t)row * ld + k0 + chunk * 8) * 2) : (int)0x80000000;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(lds + inst * 1024), 16, off, 0, 0, 0);
  }
}

// load_tile for an operand whose tile rows are scattered: lane row r of
// instruction i reads source row prow[i] (negative: a zero row), the LDS
// placement staying that of tile row r.
template <int ROWS, int BK, int NW>
__device__ __forceinline__ void load_tile_rows(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0,
                                               int kt, uint8_t* lds, int wave, int lane,
                                               const int (&prow)[ROWS / (64 / (BK / 8)) / NW]) {
  constexpr int CPR = BK / 8, RPI = 64 / CPR;
  const int rr = lane / CPR, slot = lane % CPR;
#pragma unroll
  for (int i = 0; i < ROWS / RPI / NW; ++i) {
    const int inst = wave + NW * i;
    const int row = inst * RPI + rr;
    const int chunk = swz<BK>(row, slot);
    const int off = prow[i] >= 0 && chunk * 8 < kt
                        ? (int)(((int64_t)prow[i] * ld + k0 + chunk * 8) * 2)
                        : (int)0x80000000;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(lds + inst * 1024), 16, off, 0, 0, 0);
  }
}

template <int NBW, int MBW, int BK>
__device__ __forceinline__ void load_frags(u32x4 (&af)[MBW], u32x4 (&bfr)[NBW], const uint8_t* ta,
                                           const uint8_t* tb, int wm, int wn, int lane, int ks) {
  const int chunk = 2 * ks + (lane >> 5);
  const int r32 = lane & 31;
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
    const int row = wm + i * 32 + r32;
    af[i] = *reinterpret_cast<const u32x4*>(ta + row * (BK * 2) + swz<BK>(row, chunk) * 16);
  }
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int row = wn + i * 32 + r32;
    bfr[i] = *reinterpret_cast<const u32x4*>(tb + row * (BK * 2) + swz<BK>(row, chunk) * 16);
  }
}

// Zero the elements k >= kt of the 16-byte chunk that holds k = kt in every
// row of a staged ROWS x BK tile (kt % 8 != 0).  Chunks wholly past kt were
// loaded as zeros; this one holds the padding after the last column, which
// the MFMA must not see (it may hold anything, NaN included).
template <int ROWS, int BK>
__device__ __forceinline__ void zero_k_tail(uint8_t* lds, int kt) {
  const int chunk = kt >> 3;
  for (int row = threadIdx.x; row < ROWS; row += blockDim.x) {
    u32x4* c = reinterpret_cast<u32x4*>(lds + row * (BK * 2) + swz<BK>(row, chunk) * 16);
    *c = mask_tail_nb(*c, chunk * 8, kt);
  }
}

// bf16 epilogue through LDS: the wave writes its 32*MBW x BN/2 result into
// its own LDS region (16-byte chunks XOR-swizzled by row), then reads it back
// row-contiguous, so each global store instruction writes whole 128-byte
// lines instead of 16 bytes of 32 different rows.  The operand tiles are
// dead by then (the caller has passed a barrier after the last product).
// bf16 v (8 values, packed) through the epilogue activation: act 1 gives
// silu(g) * v with g the matching 8 values of G, act 2 relu(v).  The product
// is rounded to bf16 first, as a separate activation pass would see it.
__device__ __forceinline__ u32x4 epi_act(u32x4 v, int act, u32x4 g) {
  if (act == 0) return v;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float lo = bf2f(w[e] & 0xffffu), hi = bf2f(w[e] >> 16);
    if (act == 1) {  // silu(g) = g / (1 + 2^(-g log2 e)), hardware exp2 and reciprocal
      const float glo = bf2f(gw[e] & 0xffffu), ghi = bf2f(gw[e] >> 16);
      lo *= glo * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * glo));
      hi *= ghi * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * ghi));
    } else {
      lo = lo < 0.f ? 0.f : lo;
      hi = hi < 0.f ? 0.f : hi;
    }
    w[e] = pack_bf2(lo, hi);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

template <int BN, int MBW>
__device__ __forceinline__ void store_staged(const f32x16 (&acc)[BN / 64][MBW], uint16_t* C,
                                             int64_t ldc, int mw, int nw, int M, int N,
                                             uint8_t* smem, int wave, int lane, int act = 0,
                                             const uint16_t* glu = nullptr, int64_t ldglu = 0) {
  constexpr int NBW = BN / 64, WN = BN / 2, RB = WN * 2, CPR = WN / 8, RPI = 64 / CPR;
  constexpr int WR = 32 * MBW;  // wave rows
  uint8_t* ep = smem + wave * (WR * RB);
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rl = 32 * j + (lane & 31), cl = 32 * i + 8 * q + 4 * (lane >> 5);
        const int ch = (cl >> 3) ^ (rl & (CPR - 1));
        *reinterpret_cast<u32x2*>(ep + rl * RB + ch * 16 + ((cl >> 2) & 1) * 8) =
            u32x2{pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                  pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
      }
  // the reads below take other lanes' writes: LDS runs one wave's accesses in order
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
  const int chl = lane % CPR, n = nw + chl * 8;
  if (act != 1) {
#pragma unroll 4
    for (int r0 = 0; r0 < WR; r0 += RPI) {
      const int rl = r0 + lane / CPR, m = mw + rl;
      const u32x4 v = epi_act(
          *reinterpret_cast<const u32x4*>(ep + rl * RB + ((chl ^ (rl & (CPR - 1))) * 16)), act,
          u32x4{0, 0, 0, 0});
      if (m >= M) continue;
      uint16_t* c = C + (int64_t)m * ldc + n;
      if (n + 7 < N) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(c));
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < 8 && n + e < N; ++e) c[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
    return;
  }
  // act 1: every row's 8 values of G in flight at once before the stores
  constexpr int NIT = WR / RPI;
  u32x4 gv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    gv[it] = u32x4{0, 0, 0, 0};
    const int m = mw + it * RPI + lane / CPR;
    if (m >= M) continue;
    const uint16_t* g = glu + (int64_t)m * ldglu + n;
    if (n + 7 < N) {
      gv[it] = *reinterpret_cast<const u32x4*>(g);
    } else {  // ragged tail: G's row may end before 8 elements
      uint32_t w[4] = {0, 0, 0, 0};
      for (int e = 0; e < 8 && n + e < N; ++e) w[e >> 1] |= (uint32_t)g[e] << (16 * (e & 1));
      gv[it] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int rl = it * RPI + lane / CPR, m = mw + rl;
    const u32x4 v = epi_act(
        *reinterpret_cast<const u32x4*>(ep + rl * RB + ((chl ^ (rl & (CPR - 1))) * 16)), 1,
        gv[it]);
    if (m >= M) continue;
    uint16_t* c = C + (int64_t)m * ldc + n;
    if (n + 7 < N) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(c));
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 8 && n + e < N; ++e) c[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// One 32-row block j of the wave's result through its own 32 x BN/2 LDS
// region, as in store_staged: the persistent kernel stages row block by row
// block so that the staging fits beside its operand ring.
template <int BN, int MBW>
__device__ __forceinline__ void store_block(const f32x16 (&acc)[BN / 64][MBW], int j, uint16_t* C,
                                            int64_t ldc, int mj, int nw, int M, int N,
                                            uint8_t* ep, int lane) {
  constexpr int NBW = BN / 64, WN = BN / 2, RB = WN * 2, CPR = WN / 8, RPI = 64 / CPR;
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rl = lane & 31, cl = 32 * i + 8 * q + 4 * (lane >> 5);
      const int ch = (cl >> 3) ^ (rl & (CPR - 1));
      *reinterpret_cast<u32x2*>(ep + rl * RB + ch * 16 + ((cl >> 2) & 1) * 8) =
          u32x2{pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // other lanes' writes are read below (in-order LDS)
  asm volatile("" ::: "memory");
  const int chl = lane % CPR, n = nw + chl * 8;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int rl = r0 + lane / CPR, m = mj + rl;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ep + rl * RB + ((chl ^ (rl & (CPR - 1))) * 16));
    if (m >= M) continue;
    uint16_t* c = C + (int64_t)m * ldc + n;
    if (n + 7 < N) {
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(c));
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 8 && n + e < N; ++e) c[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
  asm volatile("" ::: "memory");
}

struct BigArgs {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  void* c;        // bf16 or fp32 [M, ldc]
  int64_t ldc;
  uint16_t* c2;   // optional bf16 copy of an fp32 output [M, ldc2], 8-byte aligned rows
  int64_t ldc2;
  int M, N, K;
  int vec;        // C rows allow 16-byte (2) / 8-byte (1) stores, else element stores
  const int32_t* m_valid;  // optional live row count on the device (rows past it are skipped)
  const float* rope;       // rotary table [max_pos][hd/2] of (cos, sin), or null
  int64_t max_pos;
  const int32_t* seq_off;  // [nseq + 1] packed-row offsets: row m sits at position m - seq_off[i]
  int nseq;
  int ksplit;              // K ranges (> 1: each writes an fp32 partial to c + range * split_stride)
  int kchunk;              // elements of K per range (a multiple of 64)
  int64_t split_stride;
  int accum;               // fp32 C += the product (C read and written)
  int act;                 // bf16 C, staged stores: 1 = silu(G) * product, 2 = relu(product)
  const uint16_t* glu;     // G [M, ldglu] bf16 (act 1), 16-byte aligned rows
  int64_t ldglu;
  // Split tail (bf16 C with 16-byte row stores only; tail_n 0: none): the
  // first tail_full tiles of the list (a multiple of 256) run whole; each of
  // the last tail_n runs as tail_split K ranges of tail_kchunk elements whose
  // fp32 partials go to tail_part, summed in range order by
  // tail_reduce_kernel.  So a part-filled last round keeps every CU busy.
  int tail_full, tail_n, tail_split, tail_kchunk;
  float* tail_part;        // [tail_n][tail_split][256 * BN], accumulator order
  // Grouped launch (GROUP instances, fp32 C): gnum members side by side in N,
  // member i over column tiles [gct[i], gct[i + 1]) with its own B rows (gb,
  // gldb), C (gc, gldc), optional bf16 copy (gc2, gldc2) and width gn; b, ldb,
  // c, ldc, c2, ldc2 and N above are not used.
  int gnum;
  int gct[kMaxGemmGroup + 1];
  const uint16_t* gb[kMaxGemmGroup];
  int64_t gldb[kMaxGemmGroup];
  float* gc[kMaxGemmGroup];
  int64_t gldc[kMaxGemmGroup];
  uint16_t* gc2[kMaxGemmGroup];
  int64_t gldc2[kMaxGemmGroup];
  int gn[kMaxGemmGroup];
  int gvec[kMaxGemmGroup];  // each member's store width (as vec)
};

template <int BN, int BK>
constexpr int big_stage_bytes() { return (gBM + BN) * BK * 2; }

// LDS of one launch: the operand ring, reused by the epilogue (bf16 result
// staging 256 * BN * 2 bytes; rotary tables 256 rows * HD * 4 bytes), then
// (rotary) 2 KB of sequence offsets and row positions.
// Tile order: tiles are listed kGroupM row tiles at a time, column by column
// (tile q of the group of rows [g, g + kGroupM) is row g + q % rows, column
// q / rows).  An XCD's contiguous run of tiles is then a block of rows x
// columns, so the tiles it runs at once share both their A rows and their B
// rows in its L2 (row by row, every column tile of a row ran at once and the
// B operand streamed through the L2 again for every row).
constexpr int kGroupM = 4;
__device__ __forceinline__ int group_rows(int t, int ntn, int ntm) {
  const int first = t / (kGroupM * ntn) * kGroupM;
  const int rows = min(kGroupM, ntm - first), q = t % (kGroupM * ntn);
  return (first + q % rows) * ntn + q / rows;
}

template <int BN, int BK, int NS, int HD>
constexpr int big_lds_bytes() {
  constexpr int ring = NS * big_stage_bytes<BN, BK>();
  constexpr int ep = gBM * BN * 2 > gBM * HD * 4 ? gBM * BN * 2 : gBM * HD * 4;
  return (ring > ep ? ring : ep) + (HD > 0 ? 2048 : 0);
}

// HD > 0: rotate each head's column pairs (c, c + HD/2) of row m by the
// angles of the row's position (a wave's 128 columns hold whole heads).
// MBW: 32-row blocks per wave.  The tile's 256 rows x BN columns are split
// over 256 / (32 * MBW) x 2 waves: MBW = 4 gives 4 waves of 128 x BN/2 (one
// wave per SIMD, 512 registers), MBW = 2 gives 8 waves of 64 x BN/2 (two
// per SIMD, at most 256 registers each).
// TAIL: the launch has a split tail (a separate instance, so that launches
// without one keep the plain tile mapping and its register count).  GROUP:
// a grouped launch (the member table of BigArgs).
template <int BN, int BK, int NS, bool OUT_F32, int HD, int MBW, bool TAIL = false,
          bool GROUP = false>
__global__ __launch_bounds__(2 * 256 / (32 * MBW) * 64) void gemm_big_kernel(BigArgs p) {
  static_assert(!TAIL || (!OUT_F32 && HD == 0), "split tails: bf16 output, no rotary");
  static_assert(!GROUP || (OUT_F32 && HD == 0 && !TAIL), "grouped launches: fp32 output");
  static_assert(HD == 0 || (BN == 256 && !OUT_F32 && (HD == 64 || HD == 128)), "rotary tiles");
  static_assert((BK == 32 || BK == 64) && NS >= 2, "pipeline shape");
  static_assert(MBW == 2 || MBW == 4, "wave tile");
  constexpr int NW = 2 * gBM / (32 * MBW);  // waves
  constexpr int NBW = BN / 64;              // 32-column blocks per wave
  constexpr int kTileA = gBM * BK * 2;
  constexpr int kStage = big_stage_bytes<BN, BK>();
  constexpr int IPW = kStage / 1024 / NW;   // load instructions per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int M = p.M;
  if (p.m_valid) {  // the grid covers the capacity; spread the live tiles over the XCDs
    const int nv = *p.m_valid;
    M = nv < 0 ? 0 : (nv > p.M ? p.M : nv);
  }
  const int ntn = GROUP ? p.gct[p.gnum] : (p.N + BN - 1) / BN, ntm = (M + gBM - 1) / gBM;
  int vt, kr, kc = p.kchunk;  // list position of the tile, its K range and range length
  bool tail_unit = false;     // a K range of a split-tail tile: fp32 partial out
  if constexpr (!TAIL) {
    const int ntiles = ntn * ntm * p.ksplit;
    const int per_xcd = (ntiles + 7) / 8;
    const int v = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;  // (tile, K range)
    if ((int)blockIdx.x / 8 >= per_xcd || v >= ntiles) return;
    vt = v / p.ksplit;
    kr = v % p.ksplit;
  } else if ((int)blockIdx.x < p.tail_full) {
    // the whole tiles in XCD runs as above (tail_full is a multiple of 8)
    const int per_xcd = p.tail_full / 8;
    vt = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    kr = 0;
  } else {
    // then range kr of every tail tile, range by range (dispatched last)
    const int j = (int)blockIdx.x - p.tail_full;
    if (j >= p.tail_n * p.tail_split) return;
    vt = p.tail_full + j % p.tail_n;
    kr = j / p.tail_n;
    kc = p.tail_kchunk;
    tail_unit = true;
  }
  const int tile = group_rows(vt, ntn, ntm);
  const int m0 = (tile / ntn) * gBM;
  int n0 = (tile % ntn) * BN;  // first column of the tile (within its member's)
  // the operand and outputs of the tile (its member's in a grouped launch)
  const uint16_t* pb = p.b;
  int64_t ldb = p.ldb, ldc = p.ldc, ldc2 = p.ldc2;
  int N = p.N, vec = p.vec;
  void* pc = p.c;
  uint16_t* pc2 = p.c2;
  if constexpr (GROUP) {
    const int ct = tile % ntn;
    int mi = 0;
    while (mi + 1 < p.gnum && ct >= p.gct[mi + 1]) ++mi;
    n0 = (ct - p.gct[mi]) * BN;
    pb = p.gb[mi];
    ldb = p.gldb[mi];
    N = p.gn[mi];
    pc = p.gc[mi];
    ldc = p.gldc[mi];
    pc2 = p.gc2[mi];
    ldc2 = p.gldc2[mi];
    vec = p.gvec[mi];
  }
  const int kbeg = kr * kc, kend = min(p.K, kbeg + kc);
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(p.a + (int64_t)m0 * p.lda, view_bytes(min(M - m0, gBM), p.K, p.lda));
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(pb + (int64_t)n0 * ldb, view_bytes(min(N - n0, BN), p.K, ldb));
  const int wm = (wave >> 1) * (32 * MBW), wn = (wave & 1) * (BN / 2);
  const int nk = (kend - kbeg + BK - 1) / BK;

  int so = 0;  // rotary: this thread's entry of the sequence offsets, staged after the loop
  if (HD > 0 && (int)threadIdx.x <= p.nseq) so = p.seq_off[threadIdx.x];

  f32x16 acc[NBW][MBW];  // [n block][m block]; lane: one m row, 4 consecutive n per 4 regs
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) acc[i][j] = f32x16{};

  auto load_stage = [&](int t) {
    uint8_t* st = smem + (t % NS) * kStage;
    const int k0 = kbeg + t * BK;
    load_tile<gBM, BK, NW>(ra, p.lda, k0, kend - k0, st, wave, lane);
    load_tile<BN, BK, NW>(rb, ldb, k0, kend - k0, st + kTileA, wave, lane);
  };
  // k-tile t's loads are done once at most the stages issued after it are
  // pending (`younger` of them; vector-memory loads complete in order)
  auto wait_stage = [&](int younger) {
    if (younger >= NS - 1) wait_vm<(NS - 1) * IPW>();
    else if (NS > 3 && younger == 2) wait_vm<(NS > 3 ? 2 : 0) * IPW>();
    else if (NS > 2 && younger == 1) wait_vm<(NS > 2 ? 1 : 0) * IPW>();
    else wait_vm<0>();
  };
  // after the wait: make every wave's part of stage t visible, zeroing the
  // padding of a partial last k-tile first
  auto open_stage = [&](int t) {
    lds_barrier();
    const int kt = kend - (kbeg + t * BK);
    if (kt < BK && (kt & 7)) {
      uint8_t* st = smem + (t % NS) * kStage;
      zero_k_tail<gBM, BK>(st, kt);
      zero_k_tail<BN, BK>(st + kTileA, kt);
      lds_barrier();
    }
  };
  constexpr int KS = BK / 16;
  u32x4 af[2][MBW], bfr[2][NBW];
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nk) load_stage(t);
  wait_stage(min(NS - 2, nk - 1));
  open_stage(0);
  load_frags<NBW, MBW, BK>(af[0], bfr[0], smem, smem + kTileA, wm, wn, lane, 0);
  // One barrier per k-tile: it sits in the last k-step of tile t, after the
  // wait for tile t + 1, so the first fragments of t + 1 are read while the
  // last products of t run; it also orders every wave's reads of tile t - 1
  // before the loads that reuse its stage at the start of iteration t.  The
  // last tile is peeled so that no branch skips the barrier: the compiler's
  // LDS wait counts then stay exact (after a merge it would wait for the
  // next tile's fragments before the current products).
  auto k_tile = [&](int t, auto has_next) {
    if (t + NS - 1 < nk) load_stage(t + NS - 1);
    const uint8_t* cur = smem + (t % NS) * kStage;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int nb = (ks + 1) & 1;
      if (ks + 1 < KS) {
        load_frags<NBW, MBW, BK>(af[nb], bfr[nb], cur, cur + kTileA, wm, wn, lane, ks + 1);
      } else if constexpr (decltype(has_next)::value) {
        wait_stage(min(NS - 2, nk - 2 - t));
        open_stage(t + 1);
        const uint8_t* nxt = smem + ((t + 1) % NS) * kStage;
        load_frags<NBW, MBW, BK>(af[nb], bfr[nb], nxt, nxt + kTileA, wm, wn, lane, 0);
      }
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < MBW; ++j)
          acc[i][j] = mfma32(bfr[ks & 1][i], af[ks & 1][j], acc[i][j]);
    }
  };
  for (int t = 0; t + 1 < nk; ++t) k_tile(t, std::true_type{});
  k_tile(nk - 1, std::false_type{});
  lds_barrier();
  // (the barrier above: operand tiles dead, the epilogue may reuse the LDS)
  if constexpr (TAIL) {
    if (tail_unit) {
      // this range's partial in accumulator order, 16 bytes per lane: slot
      // ((wave, i, j, q), lane) holds acc[i][j][4q .. 4q + 3]
      f32x4* dst = reinterpret_cast<f32x4*>(
          p.tail_part + ((int64_t)(vt - p.tail_full) * p.tail_split + kr) * (gBM * BN));
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < MBW; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[((wave * NBW * MBW + i * MBW + j) * 4 + q) * 64 + lane] =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
      return;
    }
  }

  // acc[i][j] reg r -> n = wn + 32i + 8(r/4) + 4(lane/32) + r%4, m = wm + 32j + lane%32
  if constexpr (HD > 0) {
    // positions of the tile's rows from the sequence offsets (in LDS past
    // the operand buffers), then the rows' (cos, sin) tables copied straight
    // into LDS: row r's 16-byte chunk c at slot c ^ (r % CH)
    constexpr int CH = HD / 4, RPI = 64 / CH, hb = HD / 64;  // hb: partner block, + HD/2
    int* aux = reinterpret_cast<int*>(smem + big_lds_bytes<BN, BK, NS, HD>() - 2048);
    if ((int)threadIdx.x <= p.nseq) aux[threadIdx.x] = so;
    lds_barrier();
    if (threadIdx.x < gBM) {
      const int m = min(m0 + (int)threadIdx.x, M - 1);
      int lo = 0, hi = p.nseq;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (aux[mid] <= m) lo = mid; else hi = mid;
      }
      const int pos = m - aux[lo];
      aux[256 + threadIdx.x] = pos < 0 ? 0 : (pos >= p.max_pos ? (int)p.max_pos - 1 : pos);
    }
    lds_barrier();
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(p.rope, (uint64_t)p.max_pos * HD * 4);
    for (int inst = wave; inst < gBM / RPI; inst += NW) {
      const int row = inst * RPI + lane / CH, c = (lane % CH) ^ (row & (CH - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rt, (__attribute__((address_space(3))) void*)(smem + inst * 1024), 16,
          (aux[256 + row] * HD + c * 4) * 4, 0, 0, 0);
    }
    wait_vm<0>();
    lds_barrier();
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
      const int rl = wm + 32 * j + (lane & 31);
      const uint8_t* tr = smem + rl * (HD * 4);
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        if ((32 * i) % HD >= HD / 2) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int fi = (32 * i) % HD + 8 * q + 4 * (lane >> 5);  // 4 frequencies from fi
          const f32x4 cs01 =
              *reinterpret_cast<const f32x4*>(tr + ((fi / 2) ^ (rl & (CH - 1))) * 16);
          const f32x4 cs23 =
              *reinterpret_cast<const f32x4*>(tr + ((fi / 2 + 1) ^ (rl & (CH - 1))) * 16);
          const float c[4] = {cs01.x, cs01.z, cs23.x, cs23.z};
          const float sn[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a0 = acc[i][j][4 * q + e], b0 = acc[i + hb][j][4 * q + e];
            acc[i][j][4 * q + e] = a0 * c[e] - b0 * sn[e];
            acc[i + hb][j][4 * q + e] = b0 * c[e] + a0 * sn[e];
          }
        }
      }
    }
    lds_barrier();  // tables dead before the epilogue reuses the LDS
  }
  if (!OUT_F32 && vec == 2) {
    store_staged<BN, MBW>(acc, static_cast<uint16_t*>(pc), ldc, m0 + wm, n0 + wn, M, N,
                          smem, wave, lane, HD > 0 ? 0 : p.act, p.glu, p.ldglu);
    return;
  }
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
      const int m = m0 + wm + 32 * j + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn + 32 * i + 8 * q + 4 * (lane >> 5);
        const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
        const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (OUT_F32) {
          float* c = static_cast<float*>(pc) + kr * p.split_stride + (int64_t)m * ldc + n;
          uint16_t* c2 = pc2 ? pc2 + (int64_t)m * ldc2 + n : nullptr;
          if (p.accum) {
            const float v[4] = {v0, v1, v2, v3};
            if (vec == 2 && n + 3 < N) {
              const f32x4 o = *reinterpret_cast<const f32x4*>(c);
              *reinterpret_cast<f32x4*>(c) = f32x4{o.x + v0, o.y + v1, o.z + v2, o.w + v3};
            } else {
              for (int e = 0; e < 4 && n + e < N; ++e) c[e] += v[e];
            }
          } else if (vec == 2 && n + 3 < N) {
            *reinterpret_cast<f32x4*>(c) = f32x4{v0, v1, v2, v3};
            if (c2) *reinterpret_cast<u32x2*>(c2) = u32x2{pack_bf2(v0, v1), pack_bf2(v2, v3)};
          } else {
            const float v[4] = {v0, v1, v2, v3};
            for (int e = 0; e < 4 && n + e < N; ++e) {
              c[e] = v[e];
              if (c2) c2[e] = (uint16_t)f2bf(v[e]);
            }
          }
        } else {
          uint16_t* c = static_cast<uint16_t*>(pc) + (int64_t)m * ldc + n;
          if (vec >= 1 && n + 3 < N) {
            *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf2(v0, v1), pack_bf2(v2, v3)};
          } else {
            const float v[4] = {v0, v1, v2, v3};
            for (int e = 0; e < 4 && n + e < N; ++e) c[e] = (uint16_t)f2bf(v[e]);
          }
        }
      }
    }
}

// Sum of the split tail's K-range partials, in range order, into bf16 C.
// Entry e of a partial (accumulator order, 16 bytes: gemm_big_kernel's
// wave, (i, j) block, register quad q and lane) is 4 consecutive columns of
// one row.  Each thread takes 4 entries 256 apart with every range's loads in
// flight at once; a block of 1024 entries never straddles two tiles.
template <int BN, int MBW>
__global__ __launch_bounds__(256) void tail_reduce_kernel(BigArgs p) {
  constexpr int NBW = BN / 64, PER_TILE = gBM * BN / 4, CH = 4, MAXR = 4;
  static_assert(PER_TILE % (256 * CH) == 0, "whole blocks per tile");
  const int ntn = (p.N + BN - 1) / BN, ntm = (p.M + gBM - 1) / gBM;
  const int64_t first = (int64_t)blockIdx.x * (256 * CH);
  const int tt = (int)(first / PER_TILE);  // tail tile of this block
  const int tile = group_rows(p.tail_full + tt, ntn, ntm);
  const int m0 = (tile / ntn) * gBM, n0 = (tile % ntn) * BN;
  const f32x4* src = reinterpret_cast<const f32x4*>(p.tail_part) + (int64_t)tt * p.tail_split * PER_TILE;
  f32x4 v[CH][MAXR];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      const int e = (int)(first % PER_TILE) + c * 256 + (int)threadIdx.x;
      v[c][k] = k < p.tail_split ? src[(int64_t)k * PER_TILE + e] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    f32x4 sum = v[c][0];
#pragma unroll
    for (int k = 1; k < MAXR; ++k)
      if (k < p.tail_split) sum += v[c][k];
    const int e = (int)(first % PER_TILE) + c * 256 + (int)threadIdx.x;
    const int lane = e & 63, q = (e >> 6) & 3, ij = (e >> 8) % (NBW * MBW);
    const int wave = (e >> 8) / (NBW * MBW), i = ij / MBW, j = ij % MBW;
    const int m = m0 + (wave >> 1) * (32 * MBW) + 32 * j + (lane & 31);
    const int n = n0 + (wave & 1) * (BN / 2) + 32 * i + 8 * q + 4 * (lane >> 5);
    if (m >= p.M) continue;
    uint16_t* c16 = static_cast<uint16_t*>(p.c) + (int64_t)m * p.ldc + n;
    const u32x2 o{pack_bf2(sum.x, sum.y), pack_bf2(sum.z, sum.w)};
    if (n + 3 < p.N) {
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(c16));
    } else {
      const uint32_t w[2] = {o.x, o.y};
      for (int x = 0; x < 4 && n + x < p.N; ++x) c16[x] = (uint16_t)(w[x >> 1] >> (16 * (x & 1)));
    }
  }
}

// Persistent variant (bf16 output, 16-byte row stores, no rotary): one
// workgroup per CU walks its XCD's tiles x*per_xcd + w, + G/8, ... and the
// k-pipeline runs straight across tile boundaries: the next tile's first
// stages are in flight, and its first fragments in registers, while a tile's
// result leaves through LDS (one 32-row block at a time, in the LDS past the
// ring) and its stores drain behind the next tile's products.
template <int BN, int BK, int NS, int MBW>
constexpr int persist_lds_bytes() {
  return NS * big_stage_bytes<BN, BK>() + (2 * gBM / (32 * MBW)) * 32 * BN;
}

template <int BN, int BK, int NS, int MBW>
__global__ __launch_bounds__(2 * 256 / (32 * MBW) * 64) void gemm_persist_kernel(BigArgs p) {
  static_assert((BK == 32 || BK == 64) && NS >= 2 && (MBW == 2 || MBW == 4), "shape");
  constexpr int NW = 2 * gBM / (32 * MBW), NBW = BN / 64, KS = BK / 16;
  constexpr int kTileA = gBM * BK * 2;
  constexpr int kStage = big_stage_bytes<BN, BK>();
  constexpr int IPW = kStage / 1024 / NW;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int M = p.M;
  if (p.m_valid) {
    const int nv = *p.m_valid;
    M = nv < 0 ? 0 : (nv > p.M ? p.M : nv);
  }
  const int ntn = (p.N + BN - 1) / BN, ntiles = ntn * ((M + gBM - 1) / gBM);
  const int per_xcd = (ntiles + 7) / 8, wpx = (int)gridDim.x / 8;
  const int first = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
  const int end = min(((int)blockIdx.x % 8 + 1) * per_xcd, ntiles);
  if (first >= end) return;
  const int mine = (end - first + wpx - 1) / wpx;  // tiles first, first + wpx, ...
  const int nk = (p.K + BK - 1) / BK, total = mine * nk;
  const int wm = (wave >> 1) * (32 * MBW), wn = (wave & 1) * (BN / 2);
  uint8_t* ep = smem + NS * kStage + wave * (32 * BN);  // this wave's 32 x BN/2 staging

  auto load_stage = [&](int g) {
    const int tl = first + (g / nk) * wpx, t = g % nk;
    const int m0 = (tl / ntn) * gBM, n0 = (tl % ntn) * BN;
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.a + (int64_t)m0 * p.lda, view_bytes(min(M - m0, gBM), p.K, p.lda));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.b + (int64_t)n0 * p.ldb, view_bytes(min(p.N - n0, BN), p.K, p.ldb));
    uint8_t* st = smem + (g % NS) * kStage;
    load_tile<gBM, BK, NW>(ra, p.lda, t * BK, p.K - t * BK, st, wave, lane);
    load_tile<BN, BK, NW>(rb, p.ldb, t * BK, p.K - t * BK, st + kTileA, wave, lane);
  };
  auto wait_stage = [&](int younger) {
    if (younger >= NS - 1) wait_vm<(NS - 1) * IPW>();
    else if (NS > 3 && younger == 2) wait_vm<(NS > 3 ? 2 : 0) * IPW>();
    else if (NS > 2 && younger == 1) wait_vm<(NS > 2 ? 1 : 0) * IPW>();
    else wait_vm<0>();
  };
  auto open_stage = [&](int g) {
    lds_barrier();
    const int kt = p.K - (g % nk) * BK;
    if (kt < BK && (kt & 7)) {
      uint8_t* st = smem + (g % NS) * kStage;
      zero_k_tail<gBM, BK>(st, kt);
      zero_k_tail<BN, BK>(st + kTileA, kt);
      lds_barrier();
    }
  };
  f32x16 acc[NBW][MBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) acc[i][j] = f32x16{};
  u32x4 af[2][MBW], bfr[2][NBW];
#pragma unroll
  for (int g = 0; g < NS - 1; ++g)
    if (g < total) load_stage(g);
  wait_stage(min(NS - 2, total - 1));
  open_stage(0);
  load_frags<NBW, MBW, BK>(af[0], bfr[0], smem, smem + kTileA, wm, wn, lane, 0);
  // As in gemm_big_kernel: one barrier per k-tile, in its last k-step after
  // the wait for the next k-tile (here possibly the next tile's first), with
  // the last k-tile peeled.  Stores issued by an epilogue only make the later
  // load waits stricter: loads complete in order among themselves.
  auto k_tile = [&](int g, auto has_next) {
    if (g + NS - 1 < total) load_stage(g + NS - 1);
    const uint8_t* cur = smem + (g % NS) * kStage;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int nb = (ks + 1) & 1;
      if (ks + 1 < KS) {
        load_frags<NBW, MBW, BK>(af[nb], bfr[nb], cur, cur + kTileA, wm, wn, lane, ks + 1);
      } else if constexpr (decltype(has_next)::value) {
        wait_stage(min(NS - 2, total - 2 - g));
        open_stage(g + 1);
        const uint8_t* nxt = smem + ((g + 1) % NS) * kStage;
        load_frags<NBW, MBW, BK>(af[nb], bfr[nb], nxt, nxt + kTileA, wm, wn, lane, 0);
      }
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < MBW; ++j)
          acc[i][j] = mfma32(bfr[ks & 1][i], af[ks & 1][j], acc[i][j]);
    }
    if (g % nk == nk - 1) {  // tile done: store it and start the next from zero
      const int tl = first + (g / nk) * wpx;
      const int m0 = (tl / ntn) * gBM, n0 = (tl % ntn) * BN;
#pragma unroll
      for (int j = 0; j < MBW; ++j)
        store_block<BN, MBW>(acc, j, static_cast<uint16_t*>(p.c), p.ldc, m0 + wm + 32 * j,
                             n0 + wn, M, p.N, ep, lane);
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < MBW; ++j) acc[i][j] = f32x16{};
    }
  };
  for (int g = 0; g + 1 < total; ++g) k_tile(g, std::true_type{});
  k_tile(total - 1, std::false_type{});
}

// k-pipeline of the persistent launch and the fused attention: 32-deep
// k-tiles in a ring of 3 stages; wave tile 32 * gMBW rows (every launch)
constexpr int gBK = 32, gNS = 3, gMBW = 2;

// k-pipeline of the one-tile-per-workgroup launches: 64-deep k-tiles, so each
// operand row of a direct-to-LDS load is one whole 128-byte line (32-deep
// tiles fetch every line in two halves, one k-tile apart).  Three stages of
// 384 x 64 fit the LDS for 128-column tiles, two of 512 x 64 for 256-column
// tiles.
constexpr int kBigBK = 64;
template <int BN>
constexpr int big_ns() { return BN == 128 ? 3 : 2; }

// Persistent launch: one workgroup per CU (the grid is a multiple of 8 and
// at most 256), for bf16 output with 16-byte row stores and no rotary.
template <int BN>
hipError_t launch_persist(const BigArgs& a, hipStream_t st) {
  constexpr int lds = persist_lds_bytes<BN, gBK, gNS, gMBW>();
  static_assert(lds <= 160 * 1024, "LDS");
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_persist_kernel<BN, gBK, gNS, gMBW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  const int tiles = ((a.N + BN - 1) / BN) * ((a.M + gBM - 1) / gBM);
  const int grid = std::min(256, (tiles + 7) / 8 * 8);
  hipLaunchKernelGGL((gemm_persist_kernel<BN, gBK, gNS, gMBW>), dim3((unsigned)grid),
                     dim3(2 * gBM / (32 * gMBW) * 64), lds, st, a);
  return hipGetLastError();
}

template <int BN, bool OUT_F32, int HD = 0, bool TAIL = false, bool GROUP = false>
hipError_t launch_big(const BigArgs& a, hipStream_t st) {
  constexpr int kBK = kBigBK, kNS = big_ns<BN>();
  constexpr int lds = big_lds_bytes<BN, kBK, kNS, HD>();
  static_assert(lds <= 160 * 1024, "LDS");
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_big_kernel<BN, kBK, kNS, OUT_F32, HD, gMBW, TAIL, GROUP>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  const int ntn = GROUP ? a.gct[a.gnum] : (a.N + BN - 1) / BN;
  const int tiles = ntn * ((a.M + gBM - 1) / gBM) * a.ksplit;
  const int grid = TAIL ? a.tail_full + a.tail_n * a.tail_split : tiles;
  hipLaunchKernelGGL((gemm_big_kernel<BN, kBK, kNS, OUT_F32, HD, gMBW, TAIL, GROUP>),
                     dim3((unsigned)((grid + 7) / 8 * 8)), dim3(2 * gBM / (32 * gMBW) * 64), lds,
                     st, a);
  return hipGetLastError();
}

// gemm_big_kernel with a split tail (bf16 C, 16-byte row stores), then the
// tail's reduction.
template <int BN>
hipError_t launch_big_tail(const BigArgs& a, hipStream_t st) {
  if (a.tail_split > 4) return hipErrorInvalidValue;  // tail_reduce_kernel sums up to 4
  hipError_t e = launch_big<BN, false, 0, true>(a, st);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((int64_t)a.tail_n * (gBM * BN / 4) / 1024);
  hipLaunchKernelGGL((tail_reduce_kernel<BN, gMBW>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fused decode attention
// Decode attention with the reconstruction on chip: one workgroup takes a
// 256-row block of one sequence's cached rows and TT column tiles, each the
// 256 K columns of 256/HD kv heads (an item).  Tile by tile it expands the
// block's K latents into K (the large-tile k-loop over r_k), rotates and
// rounds them to bf16 as the reconstruction would store them, and scores them
// against the sequence's query heads of those kv heads.  Then it forms the
// block's softmax partials (max m, sum l) and, per query head, the p-weighted
// sum of the block's V latent rows, which it writes with m and l: the combine
// over a sequence's blocks follows and applies V_v there
// (sum_rows p (l V_v) = (sum_rows p l) V_v), so V is never formed and the
// reconstructed rows never reach HBM.
// Blocks come from blk_off (blk_off[i] = first block of sequence i).  With a
// multiple of 8 column items each XCD keeps its share of them for every
// block; with 8 / (column items) XCDs per item each takes every few blocks:
// either way the up-projection tiles an XCD reads stay in its L2 (all of
// them exceed one L2).  Otherwise the (block, column item) pairs go to the
// XCDs in contiguous runs.
constexpr int kFusedQH = 16;  // query heads per item at most

// A load instructions per lane for a 256-row tile of BK-deep k-tiles
template <int BK, int MBW>
constexpr int tile_a_loads() { return gBM / (64 / (BK / 8)) / (2 * gBM / (32 * MBW)); }

// Source rows of this lane's A load instructions for a tile of rows
// [0, nrows): row r itself, or with a row list, map[m0 + r] when that lies in
// [0, rows) (else a zero row).  Issued early, the list's loads overlap other work.
template <int BK, int MBW>
__device__ __forceinline__ void tile_rows(int (&prow)[gBM / (64 / (BK / 8)) / (2 * gBM / (32 * MBW))], const int32_t* map,
                                          int m0, int nrows, int64_t rows, int wave, int lane) {
  constexpr int NW = 2 * gBM / (32 * MBW), RPI = 64 / (BK / 8);
#pragma unroll
  for (int i = 0; i < tile_a_loads<BK, MBW>(); ++i) {
    const int row = (wave + NW * i) * RPI + lane / (BK / 8);
    int src = row < nrows ? row : -1;
    if (map && src >= 0) {
      src = map[m0 + row];
      src = src >= 0 && src < rows ? src : -1;
    }
    prow[i] = src;
  }
}

// Stage t of the ring: k-tile t of the A rows (through the row list) and of B.
template <int BN, int BK, int NS, int MBW>
__device__ __forceinline__ void ring_stage(int t, __amdgpu_buffer_rsrc_t ra, int64_t lda,
                                           __amdgpu_buffer_rsrc_t rb, int64_t ldb, int K,
                                           uint8_t* smem, int wave, int lane,
                                           const int (&prow)[gBM / (64 / (BK / 8)) / (2 * gBM / (32 * MBW))]) {
  constexpr int NW = 2 * gBM / (32 * MBW);
  constexpr int kStage = big_stage_bytes<BN, BK>();
  uint8_t* st = smem + (t % NS) * kStage;
  load_tile_rows<gBM, BK, NW>(ra, lda, t * BK, K - t * BK, st, wave, lane, prow);
  load_tile<BN, BK, NW>(rb, ldb, t * BK, K - t * BK, st + gBM * BK * 2, wave, lane);
}

// The ring fill of a k-loop (stages 0 .. NS - 2), for a caller that issues
// it early: the ring must be dead (after the previous k-loop's last barrier)
// and no other global load issued between it and tile_mainloop(filled).
template <int BN, int BK, int NS, int MBW>
__device__ __forceinline__ void tile_ring_fill(__amdgpu_buffer_rsrc_t ra, int64_t lda,
                                               __amdgpu_buffer_rsrc_t rb, int64_t ldb, int K,
                                               uint8_t* smem, int wave, int lane,
                                               const int (&prow)[gBM / (64 / (BK / 8)) / (2 * gBM / (32 * MBW))]) {
  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nk) ring_stage<BN, BK, NS, MBW>(t, ra, lda, rb, ldb, K, smem, wave, lane, prow);
}

// The A rows of the tile are rows prow[i] of the A buffer for this lane's
// i-th A load instruction (tile_rows; negative: a zero row), so the operand can
// be read in place through a row list.  filled: tile_ring_fill has issued
// the ring fill already.
template <int BN, int BK, int NS, int MBW>
__device__ __forceinline__ void tile_mainloop(f32x16 (&acc)[BN / 64][MBW],
                                              __amdgpu_buffer_rsrc_t ra, int64_t lda,
                                              __amdgpu_buffer_rsrc_t rb, int64_t ldb, int K,
                                              uint8_t* smem, int wave, int lane,
                                              const int (&prow)[gBM / (64 / (BK / 8)) / (2 * gBM / (32 * MBW))],
                                              bool filled = false) {
  constexpr int NW = 2 * gBM / (32 * MBW), NBW = BN / 64, KS = BK / 16;
  constexpr int kTileA = gBM * BK * 2;
  constexpr int kStage = big_stage_bytes<BN, BK>();
  constexpr int IPW = kStage / 1024 / NW;
  const int wm = (wave >> 1) * (32 * MBW), wn = (wave & 1) * (BN / 2);
  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) acc[i][j] = f32x16{};
  auto load_stage = [&](int t) {
    ring_stage<BN, BK, NS, MBW>(t, ra, lda, rb, ldb, K, smem, wave, lane, prow);
  };
  auto wait_stage = [&](int younger) {
    if (younger >= NS - 1) wait_vm<(NS - 1) * IPW>();
    else if (NS > 3 && younger == 2) wait_vm<(NS > 3 ? 2 : 0) * IPW>();
    else if (NS > 2 && younger == 1) wait_vm<(NS > 2 ? 1 : 0) * IPW>();
    else wait_vm<0>();
  };
  auto open_stage = [&](int t) {
    lds_barrier();
    const int kt = K - t * BK;
    if (kt < BK && (kt & 7)) {
      uint8_t* st = smem + (t % NS) * kStage;
      zero_k_tail<gBM, BK>(st, kt);
      zero_k_tail<BN, BK>(st + kTileA, kt);
      lds_barrier();
    }
  };
  u32x4 af[2][MBW], bfr[2][NBW];
  if (!filled) {
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < nk) load_stage(t);
  }
  wait_stage(min(NS - 2, nk - 1));
  open_stage(0);
  load_frags<NBW, MBW, BK>(af[0], bfr[0], smem, smem + kTileA, wm, wn, lane, 0);
  // one barrier per k-tile, the last k-tile peeled (as in gemm_big_kernel)
  auto k_tile = [&](int t, auto has_next) {
    if (t + NS - 1 < nk) load_stage(t + NS - 1);
    const uint8_t* cur = smem + (t % NS) * kStage;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int nb = (ks + 1) & 1;
      if (ks + 1 < KS) {
        load_frags<NBW, MBW, BK>(af[nb], bfr[nb], cur, cur + kTileA, wm, wn, lane, ks + 1);
      } else if constexpr (decltype(has_next)::value) {
        wait_stage(min(NS - 2, nk - 2 - t));
        open_stage(t + 1);
        const uint8_t* nxt = smem + ((t + 1) % NS) * kStage;
        load_frags<NBW, MBW, BK>(af[nb], bfr[nb], nxt, nxt + kTileA, wm, wn, lane, 0);
      }
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < MBW; ++j)
          acc[i][j] = mfma32(bfr[ks & 1][i], af[ks & 1][j], acc[i][j]);
    }
  };
  for (int t = 0; t + 1 < nk; ++t) k_tile(t, std::true_type{});
  k_tile(nk - 1, std::false_type{});
  lds_barrier();  // operand tiles dead
}

// LDS: the operand ring (reused for the row waves' latent sums), then the
// queries, scores and tile (max, sum) pairs.
template <int HD>
constexpr int fused_ring_bytes() {
  return gNS * big_stage_bytes<256, gBK>() > 4 * kFusedQH * HD * 4
             ? gNS * big_stage_bytes<256, gBK>() : 4 * kFusedQH * HD * 4;
}
// LDS of the fused attention: the operand ring, queries, scores, tile max and
// sum, then the block's rotary tables (32 offset rows and 8 base rows of HD
// floats each).
template <int HD>
constexpr int fused_lds_bytes() {
  return fused_ring_bytes<HD>() + kFusedQH * HD * 4 + kFusedQH * 256 * 4 + kFusedQH * 2 * 4 +
         40 * HD * 4;
}

template <int HD, int TT>
__global__ __launch_bounds__(512) void attn_fused_kernel(FusedAttnArgs p) {
  constexpr int BN = 256, MBW = gMBW, NBW = BN / 64;
  constexpr int QH = kFusedQH;
  constexpr int KPT = BN / HD;  // kv heads per column tile
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* qs = reinterpret_cast<float*>(smem + fused_ring_bytes<HD>());  // [QH][HD] queries
  float* ps = qs + QH * HD;                               // [QH][256] scores, then p
  float* ml = ps + QH * 256;                              // [QH][2] tile max and sum
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // an item: one block and TT adjacent column tiles (the last item of a
  // block may hold fewer)
  const int dkv = p.Hkv * HD, ntn = (dkv + BN - 1) / BN, nti = (ntn + TT - 1) / TT;
  int gb, it;
  if (nti % 8 == 0) {
    // each XCD keeps nti / 8 column items (their V_k and V_v rows stay in its
    // L2) and walks the blocks in order, its column items of a block together
    const int npx = nti / 8, w = (int)blockIdx.x / 8;
    if (w >= p.nbpad * npx) return;
    gb = w / npx;
    it = ((int)blockIdx.x % 8) * npx + w % npx;
  } else if (8 % nti == 0) {
    // 8 / nti XCDs per column item, each taking every (8 / nti)-th block: an
    // XCD keeps one item's factor rows in its L2, and a block's latent rows
    // are fetched by 8 / nti XCDs rather than by all of them
    const int xpi = 8 / nti, x = (int)blockIdx.x % 8;
    it = x % nti;
    gb = ((int)blockIdx.x / 8) * xpi + x / nti;
    if (gb >= p.nbpad) return;
  } else {
    // the (block, column item) list in contiguous runs per XCD, a block's
    // column items together
    const int nitems = p.nbpad * nti, per_xcd = (nitems + 7) / 8;
    const int item = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
    if ((int)blockIdx.x / 8 >= per_xcd || item >= nitems) return;
    gb = item / nti;
    it = item % nti;
  }
  if (gb >= p.blk_off[p.S]) return;
  int i = 0, hi = p.S;  // the sequence: the last i with blk_off[i] <= gb
  while (hi - i > 1) {
    const int mid = (i + hi) >> 1;
    if (p.blk_off[mid] <= gb) i = mid; else hi = mid;
  }
  const int beg = p.seq_off[i];
  if (beg < 0 || beg >= p.cap) return;  // offsets are device data: stay inside cap
  const int n = min(p.seq_off[i + 1], p.cap) - beg;
  const int r0 = (gb - p.blk_off[i]) * gBM;
  if (r0 < 0 || r0 >= n) return;
  const int nrows = min(gBM, n - r0), m0 = beg + r0, nt0 = it * TT;
  const int grp = p.H / p.Hkv, kv0 = nt0 * KPT;
  const int nkv = min(TT * KPT, p.Hkv - kv0), nq = nkv * grp;  // of the item
  const int wm = (wave >> 1) * (32 * MBW), wn = (wave & 1) * (BN / 2);

  // this lane's latent rows (pool rows through the remap list, or rows of the
  // compact copy), shared by the K and V expansions
  int prow[tile_a_loads<gBK, MBW>()];
  tile_rows<gBK, MBW>(prow, p.remap, m0, nrows, p.pool_rows, wave, lane);

  // the item's query heads, rotated at the new token's position and scaled
  {
    int qp = p.pos[i];
    qp = qp < 0 ? 0 : (qp >= p.max_pos ? (int)p.max_pos - 1 : qp);
    const float scale = 1.0f / sqrtf((float)HD);
    for (int t = threadIdx.x; t < nq * (HD / 2); t += blockDim.x) {
      const int ql = t / (HD / 2), e = t % (HD / 2), h = kv0 * grp + ql;
      const float cs = p.rope[((int64_t)qp * (HD / 2) + e) * 2];
      const float sn = p.rope[((int64_t)qp * (HD / 2) + e) * 2 + 1];
      const float a = bf2f(p.q[(int64_t)i * p.ldq + h * HD + e]);
      const float b = bf2f(p.q[(int64_t)i * p.ldq + h * HD + e + HD / 2]);
      qs[ql * HD + e] = (a * cs - b * sn) * scale;
      qs[ql * HD + e + HD / 2] = (b * cs + a * sn) * scale;
    }
  }
  // The block's rotary tables in LDS, for angle addition: the angle of
  // position r0 + 32k + l is that of r0 + 32k (base row k < 8) plus that of l
  // (offset row l < 32, the same for every block).  Direct-to-LDS loads,
  // issued before the K k-loop, whose first wait and barrier cover them.
  // Offset row l's 16-byte chunk c sits in slot l * CPR + (c ^ (l & 15)), so
  // the 16 lanes of a read group (16 rows at one chunk) hit distinct bank
  // slots; a base row is read by a whole half-wave at one address.  Rows past
  // the table (only rows past the sequence, whose scores are masked) take its
  // last row.
  static_assert(MBW == 2, "two 32-row blocks per wave");
  constexpr int CPR = HD / 4;  // 16-byte chunks per table row (HD / 2 (cos, sin) pairs)
  uint8_t* rope_l = reinterpret_cast<uint8_t*>(ml + QH * 2);
  {
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(p.rope, (uint64_t)p.max_pos * HD * 4);
    constexpr int NI = 40 * CPR / 64;  // load instructions: 10 (HD 64), 20 (HD 128)
    for (int inst = wave; inst < NI; inst += 8) {
      const int slot = inst * 64 + lane;
      int row, c;
      if (slot < 32 * CPR) {
        row = slot / CPR;
        c = (slot % CPR) ^ (row & 15);
      } else {
        row = r0 + 32 * ((slot - 32 * CPR) / CPR);
        c = slot % CPR;
      }
      row = min(row, (int)p.max_pos - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rt, (__attribute__((address_space(3))) void*)(rope_l + inst * 1024), 16,
          (row * HD + c * 4) * 4, 0, 0, 0);
    }
  }
  f32x16 acc[NBW][MBW];
  // the item's column tiles one after another (the ring, acc and the
  // rotary tables reused); their scores gather in ps for one softmax
#pragma nounroll
  for (int tt = 0; tt < TT; ++tt) {
    const int n0 = (nt0 + tt) * BN;
    if (n0 >= dkv) break;
    const int kt0 = tt * KPT;               // the tile's first kv head in the item
    const int nkt = min(KPT, nkv - kt0);    // its kv heads
    // K = latents . V_k^T (the first k-loop's barriers also publish qs and the
    // tables); the ring of every tile after the first was filled during the
    // previous tile's rotary and scores
    const __amdgpu_buffer_rsrc_t rkl =
        p.remap ? make_rsrc(p.kl, view_bytes(p.pool_rows, p.rk, p.ldkl))
                : make_rsrc(p.kl + (int64_t)m0 * p.ldkl, view_bytes(nrows, p.rk, p.ldkl));
    tile_mainloop<BN, gBK, gNS, MBW>(
        acc, rkl, p.ldkl,
        make_rsrc(p.vk + (int64_t)n0 * p.ldvk, view_bytes(min(dkv - n0, BN), p.rk, p.ldvk)),
        p.ldvk, p.rk, smem, wave, lane, prow, tt > 0);
    if (tt + 1 < TT && n0 + BN < dkv)
      tile_ring_fill<BN, gBK, gNS, MBW>(
          rkl, p.ldkl,
          make_rsrc(p.vk + (int64_t)(n0 + BN) * p.ldvk,
                    view_bytes(min(dkv - n0 - BN, BN), p.rk, p.ldvk)),
          p.ldvk, p.rk, smem, wave, lane, prow);
    // rotate each head's column pairs (c, c + HD/2) by the row's position (its
    // index in the sequence), then round to bf16.  acc[i][j] reg v: column
    // wn + 32i + 8(v/4) + 4(lane/32) + v%4, row wm + 32j + lane%32.
    // (cos, sin) of row wm + 32j + l from the tables: base row wm / 32 + j
    // rotated by offset row l = lane % 32.
    constexpr int hb = HD / 64;
    const int l = lane & 31;
    const uint8_t* ro = rope_l + l * CPR * 16;
    const uint8_t* rb = rope_l + (32 + wm / 32) * CPR * 16;
  #pragma unroll
    for (int ib = 0; ib < NBW; ++ib) {
      if ((32 * ib) % HD >= HD / 2) continue;
  #pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c0 = ((32 * ib) % HD + 8 * qq + 4 * (lane >> 5)) / 2;  // frequencies 2 c0 ..
        const f32x4 o01 = *reinterpret_cast<const f32x4*>(ro + ((c0 ^ (l & 15)) << 4));
        const f32x4 o23 = *reinterpret_cast<const f32x4*>(ro + (((c0 + 1) ^ (l & 15)) << 4));
        const float oc[4] = {o01.x, o01.z, o23.x, o23.z};
        const float os[4] = {o01.y, o01.w, o23.y, o23.w};
  #pragma unroll
        for (int j = 0; j < MBW; ++j) {
          const f32x4 b01 = *reinterpret_cast<const f32x4*>(rb + ((j * CPR + c0) << 4));
          const f32x4 b23 = *reinterpret_cast<const f32x4*>(rb + ((j * CPR + c0 + 1) << 4));
          const float bc[4] = {b01.x, b01.z, b23.x, b23.z};
          const float bs[4] = {b01.y, b01.w, b23.y, b23.w};
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c = fmaf(bc[e], oc[e], -bs[e] * os[e]);
            const float sn = fmaf(bs[e], oc[e], bc[e] * os[e]);
            const float a0 = acc[ib][j][4 * qq + e], b0 = acc[ib + hb][j][4 * qq + e];
            acc[ib][j][4 * qq + e] = a0 * c - b0 * sn;
            acc[ib + hb][j][4 * qq + e] = b0 * c + a0 * sn;
          }
        }
      }
    }
  #pragma unroll
    for (int ib = 0; ib < NBW; ++ib)
  #pragma unroll
      for (int j = 0; j < MBW; ++j)
  #pragma unroll
        for (int v = 0; v < 16; ++v) acc[ib][j][v] = bf2f(f2bf(acc[ib][j][v]));
    // scores: the wave's 128 columns hold HD-wide heads; a lane has half of a
    // head's columns for its rows, the partner lane (lane ^ 32) the other half
  #pragma unroll
    for (int hk = 0; hk < 128 / HD; ++hk) {
      const int kvl = (wn + hk * HD) / HD;  // kv head within the tile
      if (kvl >= nkt) continue;
      for (int g = 0; g < grp; ++g) {
        const float* qrow = qs + ((kt0 + kvl) * grp + g) * HD;
  #pragma unroll
        for (int j = 0; j < MBW; ++j) {
          float s = 0.f;
  #pragma unroll
          for (int ib = hk * (HD / 32); ib < (hk + 1) * (HD / 32); ++ib)
  #pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int d = (32 * ib) % HD + 8 * qq + 4 * (lane >> 5);
              const f32x4 qv = *reinterpret_cast<const f32x4*>(qrow + d);
              s = fmaf(acc[ib][j][4 * qq], qv.x, s);
              s = fmaf(acc[ib][j][4 * qq + 1], qv.y, s);
              s = fmaf(acc[ib][j][4 * qq + 2], qv.z, s);
              s = fmaf(acc[ib][j][4 * qq + 3], qv.w, s);
            }
          s += __shfl_xor(s, 32);
          const int row = wm + 32 * j + (lane & 31);
          if (lane < 32) ps[((kt0 + kvl) * grp + g) * 256 + row] = row < nrows ? s : -INFINITY;
        }
      }
    }
  }
  // V is never formed.  sum_rows p[q][row] (l_row V_v^T) = (sum_rows p[q][row]
  // l_row) V_v^T, so the block's partial for query head q is the p-weighted sum
  // of its V latent rows (r_v wide), and the combine applies V_v once per
  // sequence and head.  Wave w takes rows 32w .. 32w + 31, lane c the latent
  // columns 8c .. 8c + 7 of a 512-column block; heads go four at a time, and
  // the eight waves' sums meet in the ring (dead since the K k-loop).  The
  // first 8 rows are loaded before the softmax, so they arrive while it runs.
  const __amdgpu_buffer_rsrc_t rl =
      p.remap ? make_rsrc(p.vl, view_bytes(p.pool_rows, p.rv, p.ldvl))
              : make_rsrc(p.vl + (int64_t)m0 * p.ldvl, view_bytes(nrows, p.rv, p.ldvl));
  const int rlo = wave * 32;
  // source row of row rlo + lane (lanes < 32): a pool row through the remap
  // list (-1: none), or the row of the compact copy
  int src = -1;
  if (lane < 32 && rlo + lane < nrows) {
    src = rlo + lane;
    if (p.remap) {
      const int pr = p.remap[m0 + rlo + lane];
      src = pr >= 0 && pr < p.pool_rows ? pr : -1;
    }
  }
  // row r of the wave's 32 at latent column col (zero past the block, past
  // r_v, or when missing)
  auto load_row = [&](int col, int r) {
    const int sr = __builtin_amdgcn_readlane(src, r);
    const uint32_t off = sr >= 0 && col < p.rv ? (uint32_t)(((int64_t)sr * p.ldvl + col) * 2)
                                               : 0x80000000u;  // past the buffer: reads zero
    return mask_tail_nb(bload(rl, off), col, p.rv);
  };
  u32x4 cur[8], nxt[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) cur[u] = load_row(lane * 8, u);
  __syncthreads();
  // softmax partials of the tile: wave w takes query heads w, w + 8
  for (int qh = wave; qh < nq; qh += 8) {
    float* pr = ps + qh * 256;
    float sv[4], mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sv[u] = pr[lane + 64 * u];
      mx = fmaxf(mx, sv[u]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float pv = expf(sv[u] - mx);  // rows past the block: exp(-inf) = 0
      pr[lane + 64 * u] = pv;
      sum += pv;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) {
      ml[2 * qh] = mx;
      ml[2 * qh + 1] = sum;
    }
  }
  __syncthreads();  // p, m and l published
  {
    float* red = reinterpret_cast<float*>(smem);  // [8 waves][4 heads][512 columns]
    const int pw = p.rv + 2;
    // one pass: QB query heads (of those left from q0) over latent columns
    // cb .. cb + 511; a pass of two heads (the only one of a multi-head tile)
    // does half the multiply-adds of a pass of four
    auto pass = [&](int cb, int q0, auto qbc) {
      constexpr int QB = decltype(qbc)::value;
      const int col = cb + lane * 8;
      float a[QB][8];
#pragma unroll
      for (int qi = 0; qi < QB; ++qi)
#pragma unroll
        for (int e = 0; e < 8; ++e) a[qi][e] = 0.f;
      // 8 rows at a time, the next 8 in flight while these are summed (the
      // first pass's first 8 are already in flight)
      if (cb > 0 || q0 > 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) cur[u] = load_row(col, u);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < 3) {
#pragma unroll
          for (int u = 0; u < 8; ++u) nxt[u] = load_row(col, 8 * (b + 1) + u);
        }
        // p of these 8 rows for the (up to) QB heads
        float pv[QB][8];
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
          const float* pr = ps + min(q0 + qi, nq - 1) * 256 + rlo + 8 * b;
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(pr);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(pr + 4);
          const bool on = q0 + qi < nq;
          pv[qi][0] = on ? p0.x : 0.f;
          pv[qi][1] = on ? p0.y : 0.f;
          pv[qi][2] = on ? p0.z : 0.f;
          pv[qi][3] = on ? p0.w : 0.f;
          pv[qi][4] = on ? p1.x : 0.f;
          pv[qi][5] = on ? p1.y : 0.f;
          pv[qi][6] = on ? p1.z : 0.f;
          pv[qi][7] = on ? p1.w : 0.f;
        }
        // one row at a time: its 8 values widened once, used by every head
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t ww[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
          float f[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f[2 * e] = bf2f(ww[e] & 0xffffu);
            f[2 * e + 1] = bf2f(ww[e] >> 16);
          }
#pragma unroll
          for (int qi = 0; qi < QB; ++qi)
#pragma unroll
            for (int e = 0; e < 8; ++e) a[qi][e] = fmaf(pv[qi][u], f[e], a[qi][e]);
        }
        if (b < 3) {
#pragma unroll
          for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
        }
      }
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        float* rr = red + (wave * 4 + qi) * 512 + lane * 8;
        *reinterpret_cast<f32x4*>(rr) = f32x4{a[qi][0], a[qi][1], a[qi][2], a[qi][3]};
        *reinterpret_cast<f32x4*>(rr + 4) = f32x4{a[qi][4], a[qi][5], a[qi][6], a[qi][7]};
      }
      __syncthreads();
      for (int t = threadIdx.x; t < QB * 512; t += blockDim.x) {
        const int qi = t / 512, c = t % 512;
        if (q0 + qi < nq && cb + c < p.rv) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < 8; ++w) sum += red[(w * 4 + qi) * 512 + c];
          const int h = kv0 * grp + q0 + qi;
          p.part[((int64_t)gb * p.H + h) * pw + 2 + cb + c] = sum;
        }
      }
      __syncthreads();
    };
    for (int cb = 0; cb < p.rv; cb += 512)
      for (int q0 = 0; q0 < nq; q0 += 4) {
        if (nq - q0 <= 2)
          pass(cb, q0, std::integral_constant<int, 2>{});
        else
          pass(cb, q0, std::integral_constant<int, 4>{});
      }
    for (int t = threadIdx.x; t < nq; t += blockDim.x) {
      float* out = p.part + ((int64_t)gb * p.H + kv0 * grp + t) * pw;
      out[0] = ml[2 * t];
      out[1] = ml[2 * t + 1];
    }
  }
}

template <int HD, int TT>
hipError_t launch_fused_tt(const FusedAttnArgs& a, hipStream_t st) {
  constexpr int lds = fused_lds_bytes<HD>();
  static_assert(lds <= 160 * 1024, "LDS");
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fused_kernel<HD, TT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  const int64_t ntn = (a.Hkv * HD + 255) / 256, nti = (ntn + TT - 1) / TT;
  // (the layout of the kernel's item mapping: with 8 % nti == 0, 8 / nti
  // XCDs per column item each take every (8 / nti)-th block)
  const int64_t grid = nti % 8 != 0 && 8 % nti == 0
                           ? 8 * ((a.nbpad + 8 / nti - 1) / (8 / nti))
                           : (a.nbpad * nti + 7) / 8 * 8;
  hipLaunchKernelGGL((attn_fused_kernel<HD, TT>), dim3((unsigned)grid), dim3(512), lds, st, a);
  return hipGetLastError();
}

// At hd 128, four (else two) column tiles per item wherever their query heads
// fit the item's LDS (four: MHA and GQA with 2 query heads per kv head; two:
// up to 4): the latent rows' addresses, the queries and the rotary tables are
// set up once for all, one softmax serves every tile's heads, and with four
// tiles each block's latent rows are fetched by 4 XCDs rather than 8.  On the
// 7B step: 1087 us per layer with one tile, 954 with two, 936 with four, 957
// with eight.  (At hd 64 the multi-tile kernel spills.)
template <int HD>
hipError_t launch_fused(const FusedAttnArgs& a, hipStream_t st) {
  if constexpr (HD == 128) {
    const int64_t ntn = (a.Hkv * HD + 255) / 256;
    const int grp = a.Hkv > 0 ? a.H / a.Hkv : 1;
    if (ntn >= 4 && 4 * (256 / HD) * grp <= kFusedQH) return launch_fused_tt<HD, 4>(a, st);
    if (ntn >= 2 && 2 * (256 / HD) * grp <= kFusedQH) return launch_fused_tt<HD, 2>(a, st);
  }
  return launch_fused_tt<HD, 1>(a, st);
}

// Sum of the K-range partials in range order: out32 (fp32, optional) and
// out16 (bf16, optional) [M, N].  A thread takes 4 consecutive columns of
// the partials' rows (ldp, a multiple of 8, wide: columns past N are read,
// never written).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int ksplit, int64_t stride,
                                                           int64_t ldp, int M, int N,
                                                           float* __restrict__ out32,
                                                           int64_t ld32,
                                                           uint16_t* __restrict__ out16,
                                                           int64_t ld16) {
  const int64_t q = ldp / 4, n = (int64_t)M * q;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t m = e / q, c = (e % q) * 4;
    if (c >= N) continue;
    f32x4 v = *reinterpret_cast<const f32x4*>(part + m * ldp + c);
    for (int k = 1; k < ksplit; ++k) v += *reinterpret_cast<const f32x4*>(part + k * stride + m * ldp + c);
    const float w[4] = {v.x, v.y, v.z, v.w};
    for (int e2 = 0; e2 < 4 && c + e2 < N; ++e2) {
      if (out32) out32[m * ld32 + c + e2] = w[e2];
      if (out16) out16[m * ld16 + c + e2] = (uint16_t)f2bf(w[e2]);
    }
  }
}

// 2: rows of C take 16-byte stores, 1: 8-byte stores (4 elements), 0: neither.
int store_width(const void* C, int64_t ldc, int esize) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(C);
  if (a % 16 == 0 && (ldc * esize) % 16 == 0) return 2;
  return a % (4 * esize) == 0 && (ldc * esize) % (4 * esize) == 0 ? 1 : 0;
}

// Fraction of the launch's CU-rounds doing useful columns, for a tile width.
double tile_efficiency(int M, int N, int BN) {
  const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + gBM - 1) / gBM);
  const int64_t rounds = (tiles + 255) / 256;
  return (double)tiles / (rounds * 256) * ((double)N / (((N + BN - 1) / BN) * BN));
}

// Split tail of a launch of BN-wide tiles: past at least one whole round of
// 256 tiles, a last round holding at most 128 tiles splits each of them into
// up to 4 K ranges (as many as the idle CUs allow), so that round keeps
// every CU busy for a fraction of a tile's time.  n == 0: no split.
struct TailPlan {
  int full = 0, n = 0, split = 1, kchunk = 0;
};
TailPlan tail_plan(int64_t M, int64_t N, int64_t K, int BN) {
  TailPlan t;
  const int64_t tiles = ((N + BN - 1) / BN) * ((M + gBM - 1) / gBM);
  const int64_t rem = tiles % 256;
  if (tiles < 256 || rem == 0 || rem > 128 || tiles > (int64_t(1) << 30)) return t;
  const int64_t ways = std::min<int64_t>(4, 256 / rem), nkt = (K + kBigBK - 1) / kBigBK;
  const int64_t kchunk = (nkt + ways - 1) / ways * kBigBK;
  const int64_t split = (K + kchunk - 1) / kchunk;
  if (split < 2) return t;
  t.full = (int)(tiles - rem);
  t.n = (int)rem;
  t.split = (int)split;
  t.kchunk = (int)kchunk;
  return t;
}
size_t tail_bytes(const TailPlan& t, int BN) { return (size_t)t.n * t.split * gBM * BN * 4; }

// Time of one round of 256 whole tiles (one per CU) of K depth, measured on
// MI355X (bf16, 64-deep k-tiles): 6 + 25 K/1024 us at BN 256, 4 + 15.3 K/1024
// at BN 128.  A split tail costs its units' round plus the partials' round
// trip, (0.23 + 0.29 K/4096) us per MB (fitted to 1194- and 597-column stage-1
// launches of 16384 rows at K = 4096 and 11008, and 9216 x 4096 x 4096).
double round_us(int BN, int64_t K) {
  return BN == 256 ? 6.0 + 25.0 * K / 1024 : 4.0 + 15.3 * K / 1024;
}
double plain_us(int64_t M, int64_t N, int64_t K, int BN) {
  const int64_t tiles = ((N + BN - 1) / BN) * ((M + gBM - 1) / gBM);
  return (double)((tiles + 255) / 256) * round_us(BN, K);
}
double tail_us(const TailPlan& t, int BN, int64_t K) {
  const double mb = tail_bytes(t, BN) / 1e6;
  return t.full / 256 * round_us(BN, K) + round_us(BN, t.kchunk) +
         mb * (0.23 + 0.29 * K / 4096.0);
}

}  // namespace

bool gemm_big_supported(int64_t lda, int64_t ldb) {
  // 32-bit offsets within a 256-row tile; rows start on 16-byte chunks
  return lda < (int64_t(1) << 22) && ldb < (int64_t(1) << 22) && lda % 8 == 0 && ldb % 8 == 0;
}

size_t gemm_tail_bytes(int64_t M, int64_t N) {
  // K only sets how many ranges a tail tile takes (at most 4): size for 4
  const int64_t kmax = int64_t(1) << 30;
  return std::max(tail_bytes(tail_plan(M, N, kmax, 256), 256),
                  tail_bytes(tail_plan(M, N, kmax, 128), 128));
}

hipError_t gemm_nt_big(const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                       int64_t ldc, bool c_f32, uint16_t* C2, int64_t ldc2, int64_t M,
                       int64_t N, int64_t K, hipStream_t st, float* part, size_t part_bytes) {
  BigArgs a{static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, C, ldc,
            C2, ldc2, (int)M, (int)N, (int)K, store_width(C, ldc, c_f32 ? 4 : 2),
            nullptr, nullptr, 0, nullptr, 0, 1, (int)K, 0};
  const bool narrow = tile_efficiency((int)M, (int)N, 128) > tile_efficiency((int)M, (int)N, 256) + 0.05;
  if (c_f32) return narrow ? launch_big<128, true>(a, st) : launch_big<256, true>(a, st);
  if (part && a.vec == 2) {
    // a split tail where the time estimates give it a clear edge
    double best = plain_us(M, N, K, narrow ? 128 : 256);
    int bn = 0;
    TailPlan use;
    for (const int cand : {256, 128}) {
      const TailPlan t = tail_plan(M, N, K, cand);
      if (t.n == 0 || tail_bytes(t, cand) > part_bytes) continue;
      const double us = tail_us(t, cand, K);
      if (us < 0.95 * best) {
        best = us;
        bn = cand;
        use = t;
      }
    }
    if (bn) {
      a.tail_full = use.full;
      a.tail_n = use.n;
      a.tail_split = use.split;
      a.tail_kchunk = use.kchunk;
      a.tail_part = part;
      return bn == 128 ? launch_big_tail<128>(a, st) : launch_big_tail<256>(a, st);
    }
  }
  return narrow ? launch_big<128, false>(a, st) : launch_big<256, false>(a, st);
}

int64_t gemm_group_tiles(const int64_t* N, int n, int64_t M) {
  int64_t cols = 0;
  for (int i = 0; i < n; ++i) cols += (N[i] + 127) / 128;
  return cols * ((M + gBM - 1) / gBM);
}

hipError_t gemm_nt_big_group(const void* A, int64_t lda, const GemmMember* g, int n, int64_t M,
                             int64_t K, hipStream_t st) {
  if (n < 1 || n > kMaxGemmGroup) return hipErrorInvalidValue;
  BigArgs a{static_cast<const uint16_t*>(A), lda, nullptr, 0, nullptr, 0, nullptr, 0, (int)M, 0,
            (int)K, 2, nullptr, nullptr, 0, nullptr, 0, 1, (int)K, 0};
  a.gnum = n;
  a.gct[0] = 0;
  for (int i = 0; i < n; ++i) {
    a.gb[i] = static_cast<const uint16_t*>(g[i].B);
    a.gldb[i] = g[i].ldb;
    a.gc[i] = g[i].C;
    a.gldc[i] = g[i].ldc;
    a.gc2[i] = g[i].C2;
    a.gldc2[i] = g[i].ldc2;
    a.gn[i] = (int)g[i].N;
    a.gct[i + 1] = a.gct[i] + (int)((g[i].N + 127) / 128);
    // 16-byte fp32 stores and 8-byte copies where the member's rows allow them
    const bool c2ok = !g[i].C2 || (reinterpret_cast<uintptr_t>(g[i].C2) % 8 == 0 && g[i].ldc2 % 4 == 0);
    a.gvec[i] = store_width(g[i].C, g[i].ldc, 4) == 2 && c2ok ? 2 : 0;
  }
  return launch_big<128, true, 0, false, true>(a, st);
}

int gemm_split_ranges(int64_t M, int64_t N, int64_t K) {
  // K ranges for a launch whose 128-column tiles leave most CUs idle: enough
  // ranges for ~256 workgroups, each range at least 512 deep
  const int64_t tiles = ((N + 127) / 128) * ((M + gBM - 1) / gBM);
  if (tiles >= 128 || K < 1024) return 1;
  // one workgroup per CU: more ranges would leave some CUs with two
  int64_t s = 256 / tiles;
  s = std::min<int64_t>(s, 8);
  s = std::min<int64_t>(s, K / 512);
  return (int)std::max<int64_t>(s, 1);
}

size_t gemm_split_bytes(int64_t M, int64_t N) {
  // the largest partial buffer any K of this M, N can ask for
  const int64_t tiles = ((N + 127) / 128) * ((M + gBM - 1) / gBM);
  if (tiles >= 128) return 0;
  const int64_t s = std::min<int64_t>(256 / tiles, 8);
  return (size_t)s * M * ((N + 7) / 8 * 8) * 4;
}

hipError_t attn_fused_decode(const FusedAttnArgs& a, int hd, hipStream_t st) {
  if (hd == 128) return launch_fused<128>(a, st);
  if (hd == 64) return launch_fused<64>(a, st);
  return hipErrorInvalidValue;
}

hipError_t gemm_nt_big_act(const void* A, int64_t lda, const void* B, int64_t ldb, uint16_t* C,
                           int64_t ldc, int act, const uint16_t* G, int64_t ldg, int64_t M,
                           int64_t N, int64_t K, hipStream_t st) {
  const bool g_ok = act != 1 || (G && reinterpret_cast<uintptr_t>(G) % 16 == 0 && ldg % 8 == 0);
  if (act < 1 || act > 2 || store_width(C, ldc, 2) != 2 || !g_ok) return hipErrorInvalidValue;
  BigArgs a{static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, C, ldc,
            nullptr, 0, (int)M, (int)N, (int)K, 2, nullptr, nullptr, 0, nullptr, 0, 1, (int)K, 0,
            0, act, G, ldg};
  const bool narrow = tile_efficiency((int)M, (int)N, 128) > tile_efficiency((int)M, (int)N, 256) + 0.05;
  return narrow ? launch_big<128, false>(a, st) : launch_big<256, false>(a, st);
}

hipError_t gemm_nt_big_acc(const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                           int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  BigArgs a{static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, C, ldc,
            nullptr, 0, (int)M, (int)N, (int)K, store_width(C, ldc, 4), nullptr, nullptr, 0,
            nullptr, 0, 1, (int)K, 0, 1};
  const bool narrow = tile_efficiency((int)M, (int)N, 128) > tile_efficiency((int)M, (int)N, 256) + 0.05;
  return narrow ? launch_big<128, true>(a, st) : launch_big<256, true>(a, st);
}

hipError_t gemm_nt_big_split(const void* A, int64_t lda, const void* B, int64_t ldb, float* part,
                             float* out32, int64_t ld32, uint16_t* out16, int64_t ld16,
                             int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int ks = gemm_split_ranges(M, N, K);
  const int64_t ldp = (N + 7) / 8 * 8;
  const int kchunk = (int)(((K + ks - 1) / ks + 63) / 64 * 64);
  const int nsplit = (int)((K + kchunk - 1) / kchunk);
  BigArgs a{static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, part, ldp,
            nullptr, 0, (int)M, (int)N, (int)K, store_width(part, ldp, 4), nullptr, nullptr, 0,
            nullptr, 0, nsplit, kchunk, M * ldp};
  hipError_t e = launch_big<128, true>(a, st);
  if (e != hipSuccess) return e;
  const int64_t n = M * (ldp / 4);
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(split_reduce_kernel, dim3(blocks), dim3(256), 0, st, part, nsplit, M * ldp,
                     ldp, (int)M, (int)N, out32, ld32, out16, ld16);
  return hipGetLastError();
}

hipError_t gemm_nt_big_rows(const void* A, int64_t lda, const void* B, int64_t ldb, uint16_t* C,
                            int64_t ldc, int64_t M, const int32_t* m_valid, int64_t N, int64_t K,
                            const BigRope* rope, hipStream_t st) {
  BigArgs a{static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb, C, ldc,
            nullptr, 0, (int)M, (int)N, (int)K, store_width(C, ldc, 2), m_valid, nullptr, 0,
            nullptr, 0, 1, (int)K, 0};
  // without rotary: the persistent kernel (its stores drain behind the next
  // tile's products; worth it where the output is large against K)
  if (!rope) return a.vec == 2 ? launch_persist<256>(a, st) : launch_big<256, false>(a, st);
  if (rope->nseq < 1 || rope->nseq > 255 || rope->max_pos < 1 ||
      rope->max_pos * rope->hd * 4 >= (int64_t(1) << 31) || N % rope->hd)
    return hipErrorInvalidValue;
  a.rope = rope->table;
  a.max_pos = rope->max_pos;
  a.seq_off = rope->seq_off;
  a.nseq = rope->nseq;
  if (rope->hd == 128) return launch_big<256, false, 128>(a, st);
  if (rope->hd == 64) return launch_big<256, false, 64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lr
