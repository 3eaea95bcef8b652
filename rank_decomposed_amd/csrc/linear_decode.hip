// Decode path of the decomposed linear (few token rows, HBM-bound).
//
// DeInfer/en §2.A: the downward projection forms the rank-r intermediate,
// the upward projection maps it back.  With T <= 64 tokens both stages are
// bound by streaming U_r and V_r from HBM once.  Each stage is a skinny
// product  C[T, N] = A[T, K] . B[N, K]^T  (B = weight rows, K contiguous) on
// bf16 MFMA 16x16x32, the token dimension padded to 16 / 32 / 64: MFMA issue
// is nearly free next to the HBM stream and it avoids the VALU ceiling of a
// dot-product GEMV once T grows past ~16.
//
// Weights come row-major or fragment-packed (each 16-row x 32-column step
// stored as the 1 KiB the matrix cores consume, so a wave streams contiguous
// memory; row-major steps touch 16 rows x 64 B per load, which costs a third
// of the HBM rate on long rows).
//
// One kernel per projection; the grid holds every stage-1 tile and then every
// stage-2 tile, tile = blockIdx.x.  Workgroups are dispatched in index order
// and stage-1 tiles never wait, so a waiting stage-2 tile can never hold
// resources that a stage-1 tile it waits for still needs.
//   Every tile is one workgroup of 16 waves on a block of weight rows over a
//   K range: the waves split the range into contiguous runs and their
//   partial products meet in a fixed-order tree through LDS.
//   stage-1 tile: 16*RB1 rows of U_r^T over one of S1 K ranges (S1 > 1 only
//     where a row block alone would give a workgroup more bytes than it
//     streams quickly).  With S1 > 1 the partials meet in the workspace and
//     the last tile of the row block to arrive sums them in K-range order.
//     The finishing tile publishes its rows of t (fp32 for t_io, bf16 for
//     stage 2 in the fragment-packed layout the weights use; for T <= 16 also
//     the bf16 residual t - bf16(t), so stage 2 sees ~16 mantissa bits at the
//     cost of a second MFMA) and bumps the "t ready" counter; the last one
//     raises the GO flag.
//   stage-2 tile: 16*RB2 rows of V_r^T over all of r.  Each wave issues the
//     loads of its first PF steps of V_r *before* waiting for GO, so the V_r
//     stream overlaps stage 1; then it reads t and finishes, writing y in
//     bf16 (or adding into an fp32 accumulator).
// Synchronisation avoids cache-wide operations and hot addresses:
//   * data that crosses workgroups (partials, t) is written with
//     device-coherent stores and the writer waits for their completion before
//     it bumps a counter; readers use device-coherent loads, so neither side
//     writes back or invalidates a cache;
//   * device-scope atomics on one address serialise (~10 ns each on this
//     part), so a tile issues at most two, and waiting tiles poll the GO flag,
//     which only the last producer writes.
// Counters live in the workspace and return to zero within the call: the
// last arrival of each row block clears its counter, the last stage-1 tile
// clears the ready counter, and the last stage-2 tile past the wait clears
// GO and the stage-2 counter, so consecutive calls (and graph replays) need
// no memset.  Every wait is bounded: past ~1 s it records an error flag and
// proceeds.
#include <algorithm>
#include <mutex>

#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint32_t kOutside = 0x80000000u;  // past every buffer (tiles stay < 2 GiB)
constexpr int kCoherentLoad = 16;           // buffer-load cache policy: device scope
constexpr int kMaxGroup = 8;                // linears per launch
constexpr int kRedBudget1 = 159 * 1024;     // LDS for parked partials: one workgroup per CU
constexpr int kRedBudget2 = 79 * 1024;      //   two workgroups per CU

// One control block (uint32 words) per linear of a launch, all of them at
// the start of the workspace: each hot word on a cache line of its own, then
// one arrival counter per stage-1 row block.  Their place and size are the
// same for every call, so that data of one call never lands on words another
// call (of another shape or group size, same workspace) takes as zeroed
// counters.
enum { CTL_TREADY = 0, CTL_GO = 32, CTL_DONE2 = 64, CTL_ERR = 96, CTL_CNT = 128,
       CTL_WORDS = 4096 };

// One linear of a launch.
struct LinArgs {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* ut;
  int64_t ldu;  // row pitch in elements, or block pitch in steps when packed
  const uint16_t* vt;
  int64_t ldv;
  uint16_t* y;
  int64_t ldy;
  float* yacc;  // optional: yacc[T, ldacc] += y (fp32) instead of writing y
  int64_t ldacc;
  float* t32;  // optional fp32 t [T, ldt32] (stage-1 output)
  int64_t ldt32;
  uint16_t* thi;  // bf16 t, fragment-packed (tpack), ldtb k-steps per token block
  uint16_t* tlo;  // bf16 residual (T <= 16)
  int64_t ldtb;
  float* part;    // stage-1 split-K partials
  uint32_t* ctl;  // control block
  int d_in, r, d_out;
  int nb1, S1, kc1;  // stage-1 row blocks, K ranges per block, K range width
  int n2;            // stage-2 tiles
  int rb2;           // stage-2 tile height in 16-row blocks
  int first1, first2;  // index of the linear's first stage-1 / stage-2 tile
  int wait;          // stage-2 tiles wait for the stage-1 tiles of this launch
  int packed;        // weights fragment-packed
};

// A launch: up to kMaxGroup independent linears over the same T token rows;
// every stage-1 tile of every linear comes before every stage-2 tile.
struct DecArgs {
  LinArgs lin[kMaxGroup];
  int n, T, n1;  // linears, tokens, stage-1 tiles in all
};

// Element (tok, n) of the bf16 t handed to stage 2, which is stored
// fragment-packed like the weights: 16-token blocks of nst 32-wide steps, the
// 16 bytes of lane (tok % 16) + 16 * (n % 32 / 8) of step n / 32 holding
// n % 8.  A stage-2 fragment load is then 1 KB of contiguous memory; t in
// token rows would give 16 rows x 64 bytes, every cache line fetched in two
// halves one k-step apart.
__device__ __forceinline__ int64_t tpack(int tok, int n, int64_t nst) {
  return ((((int64_t)(tok >> 4) * nst + (n >> 5)) * 64 + (tok & 15) + 16 * ((n & 31) >> 3)) << 3) +
         (n & 7);
}
// Relaxed device-scope atomics: on gfx950 these are plain loads/stores with
// device coherence (no cache maintenance); ordering is made explicit with a
// wait for outstanding memory operations before a counter is bumped.
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_relaxed(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until every memory operation this wave issued has completed
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }
// workgroup barrier for LDS exchange only: waits for this wave's LDS
// operations (lgkmcnt 0; vmcnt and expcnt left at their maxima) but not for
// its global memory operations, unlike __syncthreads
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// NB fragments of one k-step at byte offset step_off from the per-lane bases
// off[]; a dead step goes to an offset outside the buffer (reads zero, no
// memory access).  COH selects device-coherent loads.
template <int NB, bool COH>
__device__ __forceinline__ void frag_load_at(u32x4 (&f)[NB], __amdgpu_buffer_rsrc_t rs,
                                             const uint32_t (&off)[NB], uint32_t step_off,
                                             bool live) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int o = (int)(live ? off[nb] + step_off : kOutside);
    f[nb] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, COH ? kCoherentLoad : 0));
  }
}

// Weight operand of one tile: rows [row0, row0 + 16*RB) over K range
// [kbeg, kend) (kbeg a multiple of 32), as a buffer based at the tile's first
// element plus per-lane fragment offsets and the byte stride of one k-step.
template <int RB>
struct WeightTile {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[RB];
  uint32_t step;
  __device__ WeightTile(const uint16_t* B, int64_t ld, bool packed, int N, int row0, int kbeg,
                        int kend, int lane) {
    const int ksteps = (kend - kbeg + 31) / 32;
    if (packed) {
      // fragment (block b, step s) at ((b*ld + s)*64 + lane)*16 bytes
      const int b0 = row0 / 16, nb = min(RB, (N + 15) / 16 - b0);
      rs = make_rsrc(B + ((int64_t)b0 * ld + kbeg / 32) * 512,
                     ((uint64_t)(nb - 1) * ld + ksteps) * 1024);
#pragma unroll
      for (int r = 0; r < RB; ++r) off[r] = (uint32_t)((r * ld * 64 + lane) * 16);
      step = 1024;
    } else {
      rs = make_rsrc(B + (int64_t)row0 * ld + kbeg,
                     view_bytes(min(N - row0, 16 * RB), kend - kbeg, ld));
#pragma unroll
      for (int r = 0; r < RB; ++r)
        off[r] = (uint32_t)(((r * 16 + (lane & 15)) * ld + (lane >> 4) * 8) * 2);
      step = 64;
    }
  }
};

// This wave's share of one tile: weight rows [row0, row0 + 16*RB) against
// A[0:T, kbeg:kend), over the wave's contiguous run of 32-wide k-steps.  Per
// round the wave issues the weight loads, then the activation loads, then
// the MFMAs.  Rows past T or N and steps past the wave's run fall outside
// the buffers and read zero, so the step loop has no branches; only a ragged
// last step (K range not a multiple of 32) is masked, after the loop.
// A stage-2 tile (WAIT) first issues the weight loads of its first PF steps,
// then waits for GO, then reads t with device-coherent loads.
// acc[tb][rb] lane l holds C[token tb*16 + 4*(l>>4) + v][row row0 + rb*16 + (l&15)].
template <int TB, int RB, int KSW, int PF, bool SPLIT, bool WAIT>
__device__ void tile_product(f32x4 (&acc)[TB][RB], const uint16_t* __restrict__ A,
                             const uint16_t* __restrict__ Alo, int64_t lda,
                             const uint16_t* __restrict__ B, int64_t ldb, bool packed, int T,
                             int N, int row0, int kbeg, int kend, uint32_t* ctl, bool wait,
                             float* stage = nullptr) {
  static_assert(!WAIT || PF % KSW == 0, "the prefetched steps are consumed KSW at a time");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kq = (lane >> 4) * 8;
  const int K = kend - kbeg;
  const WeightTile<RB> w(B, ldb, packed, N, row0, kbeg, kend, lane);
  // stage 2 (WAIT) reads t fragment-packed (lda = steps per token block, the
  // K range starts at 0): one k-step is 1 KB per token block
  constexpr int ASTEP = WAIT ? 1024 : 64;
  const uint64_t abytes =
      WAIT ? (uint64_t)TB * lda * 1024 : view_bytes(min(T, 16 * TB), K, lda);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(WAIT ? A : A + kbeg, abytes);
  const __amdgpu_buffer_rsrc_t ral = make_rsrc((SPLIT ? Alo : A) + (WAIT ? 0 : kbeg), abytes);
  uint32_t aoff[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)  // (packed t: lanes of tokens >= T read zero, no memory)
    aoff[tb] = WAIT ? (tb * 16 + (lane & 15) < T ? (uint32_t)((tb * lda * 64 + lane) * 16)
                                                  : kOutside)
                    : (uint32_t)(((tb * 16 + (lane & 15)) * lda + kq) * 2);

  const int nsteps = (K + 31) / 32;
  const int nfull = K / 32;
  // Stage-1 activations go through LDS (XL) for T > 16: a round of two
  // k-steps is one whole 128-byte line per token row, so waves take even
  // runs of steps.  (The MFMA fragment of one k-step is 16 token rows x 64
  // bytes; loaded straight from the caller's row-major x, every line was
  // fetched in two halves.)
  constexpr bool XL = !WAIT && !SPLIT && TB >= 2 && KSW % 2 == 0;
  const int per = XL ? 2 * ((nsteps + 2 * kWaves - 1) / (2 * kWaves))
                     : (nsteps + kWaves - 1) / kWaves;  // contiguous k-steps per wave
  const int s_lo = min(nsteps, wave * per);
  const int s_hi = min(nsteps, s_lo + per);
  const int s_full = min(s_hi, nfull);

#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[tb][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // KSW steps whose weights are in bv: load the activations, multiply
  auto round = [&](const u32x4 (*bv)[RB], int sb) {
    u32x4 av[KSW][TB], alv[KSW][TB];
    if constexpr (XL) {
      // per pair of steps: 2*TB loads of 8 token rows x 128 bytes (whole
      // lines) into the wave's own LDS region (the slot it later parks its
      // partial products in), the rows' 16-byte chunks XOR-swizzled by row;
      // then the MFMA fragments read back from it.  Only this wave touches
      // the region, so LDS ordering within the wave is all it needs.
      uint8_t* xs = reinterpret_cast<uint8_t*>(stage) + wave * (TB * 2048);
#pragma unroll
      for (int pr = 0; pr < KSW / 2; ++pr) {
        const int sp = sb + 2 * pr;
        u32x4 ld[2 * TB];
#pragma unroll
        for (int q = 0; q < 2 * TB; ++q) {
          const int row = 8 * q + (lane >> 3), c = lane & 7;
          const bool live = sp + (c >> 2) < s_full;
          ld[q] = bload(ra, live ? (uint32_t)((row * lda + sp * 32 + c * 8) * 2) : kOutside);
        }
#pragma unroll
        for (int q = 0; q < 2 * TB; ++q) {
          const int row = 8 * q + (lane >> 3), c = lane & 7;
          *reinterpret_cast<u32x4*>(xs + row * 128 + ((c ^ (row & 7)) << 4)) = ld[q];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            const int row = tb * 16 + (lane & 15), c = 4 * i + (lane >> 4);
            av[2 * pr + i][tb] =
                *reinterpret_cast<const u32x4*>(xs + row * 128 + ((c ^ (row & 7)) << 4));
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < KSW; ++i) {
        frag_load_at<TB, WAIT>(av[i], ra, aoff, (sb + i) * ASTEP, sb + i < s_full);
        if (SPLIT) frag_load_at<TB, WAIT>(alv[i], ral, aoff, (sb + i) * ASTEP, sb + i < s_full);
      }
    }
#pragma unroll
    for (int i = 0; i < KSW; ++i)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          acc[tb][r] = mfma16x16x32(av[i][tb], bv[i][r], acc[tb][r]);
          if (SPLIT) acc[tb][r] = mfma16x16x32(alv[i][tb], bv[i][r], acc[tb][r]);
        }
  };

  int s0 = s_lo;
  if (WAIT) {
    u32x4 bp[PF][RB];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      frag_load_at<RB, false>(bp[i], w.rs, w.off, (s_lo + i) * w.step, s_lo + i < s_full);
    if (wait && threadIdx.x == 0) {
      uint32_t spins = 0;
      while (load_relaxed(ctl + CTL_GO) == 0u) {
        __builtin_amdgcn_s_sleep(8);
        if (++spins > kSpinLimit) {
          store_relaxed(ctl + CTL_ERR, 1u);
          break;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i0 = 0; i0 < PF; i0 += KSW) round(bp + i0, s_lo + i0);
    s0 = s_lo + PF;
  }
  for (; s0 < s_full; s0 += KSW) {
    u32x4 bv[KSW][RB];
#pragma unroll
    for (int i = 0; i < KSW; ++i)
      frag_load_at<RB, false>(bv[i], w.rs, w.off, (s0 + i) * w.step, s0 + i < s_full);
    round(bv, s0);
  }
  if (nfull < nsteps && nfull >= s_lo && nfull < s_hi) {
    // ragged last step of the K range, owned by this wave
    const int kk = nfull * 32 + kq;
    u32x4 bv[RB], av[TB], alv[TB];
    frag_load_at<RB, false>(bv, w.rs, w.off, nfull * w.step, true);
    frag_load_at<TB, WAIT>(av, ra, aoff, nfull * ASTEP, true);
    if (SPLIT) frag_load_at<TB, WAIT>(alv, ral, aoff, nfull * ASTEP, true);
#pragma unroll
    for (int r = 0; r < RB; ++r) bv[r] = mask_tail_nb(bv[r], kk, K);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      av[tb] = mask_tail_nb(av[tb], kk, K);
      if (SPLIT) alv[tb] = mask_tail_nb(alv[tb], kk, K);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        acc[tb][r] = mfma16x16x32(av[tb], bv[r], acc[tb][r]);
        if (SPLIT) acc[tb][r] = mfma16x16x32(alv[tb], bv[r], acc[tb][r]);
      }
  }
}

// LDS slots for parking a tile of NR accumulator registers per lane: one
// per wave when 16 x NR x 256 bytes fit the budget, else 8 (waves w and
// w + 8 added in registers first).
constexpr int park_slots(int NR, int lds_budget) { return 16 * NR * 256 <= lds_budget ? 16 : 8; }

// Copy this wave's accumulators into LDS slot `slot` as red[slot][reg][lane].
template <int TB, int RB>
__device__ __forceinline__ void park_slot(const f32x4 (&acc)[TB][RB], float* red, int slot) {
  constexpr int NR = TB * RB * 4;
  float* b = red + slot * NR * 64 + (threadIdx.x & 63);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) b[((tb * RB + r) * 4 + v) * 64] = acc[tb][r][v];
}

// Park the 16 waves' partial products in NSLOT slots whose sum is the tile.
template <int TB, int RB, int NSLOT>
__device__ __forceinline__ void park(f32x4 (&acc)[TB][RB], float* red) {
  const int wave = threadIdx.x >> 6;
  if (NSLOT == kWaves) {
    park_slot<TB, RB>(acc, red, wave);
    lds_barrier();
    return;
  }
  constexpr int NR = TB * RB * 4;
  if (wave >= 8) park_slot<TB, RB>(acc, red, wave - 8);
  lds_barrier();
  if (wave < 8) {
    const float* b = red + wave * NR * 64 + (threadIdx.x & 63);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[tb][r][v] += b[((tb * RB + r) * 4 + v) * 64];
  }
  lds_barrier();
  if (wave < 8) park_slot<TB, RB>(acc, red, wave);
  lds_barrier();
}

// Element e of a parked tile summed over the slots, pairwise in a fixed order
// (slot w + 8 -- already added in registers when there are 8 slots -- then
// + 4, + 2, + 1: the same order either way).
template <int NR, int NSLOT>
__device__ __forceinline__ float sum_waves(const float* red, int e) {
  float v[NSLOT];
#pragma unroll
  for (int w = 0; w < NSLOT; ++w) v[w] = red[w * NR * 64 + e];
#pragma unroll
  for (int h = NSLOT / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int w = 0; w < h; ++w) v[w] += v[w + h];
  return v[0];
}

// Element e = reg*64 + lane of a tile -> token and row offset (MFMA 16x16
// accumulator layout, reg = (tb*RB + rb)*4 + v).
template <int RB>
__device__ __forceinline__ void elem_coords(int e, int* tok, int* row) {
  const int reg = e >> 6, lane = e & 63;
  const int v = reg & 3, rb = (reg >> 2) % RB, tb = (reg >> 2) / RB;
  *tok = tb * 16 + 4 * (lane >> 4) + v;
  *row = rb * 16 + (lane & 15);
}

// One stage-2 tile: 16*RB2 rows of V_r^T over all of r, then y.
template <int TB, int RB2, int KSW2, int PF, bool SPLIT, int BUDGET>
__device__ __forceinline__ void stage2_tile(const LinArgs& p, int T, int tile, float* red) {
  constexpr int NR = TB * RB2 * 4, NE = NR * 64;
  constexpr int EPT = (NE + kThreads - 1) / kThreads;
  const int row0 = (tile - p.first2) * 16 * RB2;
  f32x4 acc[TB][RB2];
  tile_product<TB, RB2, KSW2, PF, SPLIT, true>(acc, p.thi, p.tlo, p.ldtb, p.vt, p.ldv,
                                               p.packed != 0, T, p.d_out, row0, 0, p.r,
                                               p.ctl, p.wait != 0);
  // count this tile past the wait; the last one clears GO for the next call.
  // The LDS barrier does not wait for global memory, so this contended
  // atomic's round trip overlaps the reduction.
  uint32_t old = 0;
  if (p.wait && threadIdx.x == 0) old = atomic_add_agent(p.ctl + CTL_DONE2, 1u);
  constexpr int NS = park_slots(NR, BUDGET);
  park<TB, RB2, NS>(acc, red);
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = threadIdx.x + i * kThreads;
    int tok, ro;
    elem_coords<RB2>(e, &tok, &ro);
    const int n = row0 + ro;
    if (e >= NE || tok >= T || n >= p.d_out) continue;
    const float val = sum_waves<NR, NS>(red, e);
    if (p.yacc)
      p.yacc[(int64_t)tok * p.ldacc + n] += val;  // each element owned by one tile
    else
      p.y[(int64_t)tok * p.ldy + n] = (uint16_t)f2bf(val);
  }
  if (p.wait && threadIdx.x == 0 && old == (uint32_t)(p.n2 - 1)) {
    store_relaxed(p.ctl + CTL_GO, 0u);
    store_relaxed(p.ctl + CTL_DONE2, 0u);
  }
}

template <int TB, int RB1, int RB2, int RB2L, int KSW1, int KSW2, int KSW2L, int PF, int PFL,
          bool SPLIT, int WG_PER_CU>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4 * WG_PER_CU, 4 * WG_PER_CU)))
void decode_kernel(DecArgs args) {
  extern __shared__ __attribute__((aligned(16))) float red[];  // [slots][NR][64], + padding
  constexpr int kBudget = WG_PER_CU == 1 ? kRedBudget1 : kRedBudget2;
  __shared__ uint32_t sh_last;
  const int tile = (int)blockIdx.x;
  const int T = args.T;

  if (tile < args.n1) {
    int li = 0;  // the linear owning this stage-1 tile (workgroup-uniform)
    while (li + 1 < args.n && tile >= args.lin[li + 1].first1) ++li;
    const LinArgs& p = args.lin[li];
    constexpr int NR = TB * RB1 * 4, NE = NR * 64;
    constexpr int EPT = (NE + kThreads - 1) / kThreads;  // elements per thread
    const int t1 = tile - p.first1;
    const int blk = t1 / p.S1, s = t1 % p.S1;
    const int row0 = blk * 16 * RB1;
    const int kbeg = s * p.kc1, kend = min(p.d_in, kbeg + p.kc1);
    f32x4 acc[TB][RB1];
    tile_product<TB, RB1, KSW1, KSW1, false, false>(acc, p.x, nullptr, p.ldx, p.ut, p.ldu,
                                                    p.packed != 0, T, p.r, row0, kbeg, kend,
                                                    p.ctl, false, red);
    constexpr int NS = park_slots(NR, kBudget);
    park<TB, RB1, NS>(acc, red);
    float val[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = threadIdx.x + i * kThreads;
      val[i] = e < NE ? sum_waves<NR, NS>(red, e) : 0.f;
    }
    if (p.S1 > 1) {
      // the K ranges of the row block meet in the workspace; the last to
      // arrive sums them in K-range order (loads a few partials at a time so
      // that their round trips overlap)
      float* base = p.part + (int64_t)blk * p.S1 * NE + threadIdx.x;
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (threadIdx.x + i * kThreads < NE) store_coherent(base + (int64_t)s * NE + i * kThreads, val[i]);
      wait_memory();
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t old = atomic_add_agent(p.ctl + CTL_CNT + blk, 1u);
        sh_last = old == (uint32_t)(p.S1 - 1);
        if (sh_last) store_relaxed(p.ctl + CTL_CNT + blk, 0u);  // every sibling has arrived
      }
      __syncthreads();
      if (!sh_last) return;
      constexpr int JB = 8;
#pragma unroll
      for (int i = 0; i < EPT; ++i) val[i] = 0.f;
      for (int j0 = 0; j0 < p.S1; j0 += JB) {
        float l[JB][EPT];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int i = 0; i < EPT; ++i)
            l[jj][i] = threadIdx.x + i * kThreads < NE
                           ? load_coherent(base + (int64_t)min(j0 + jj, p.S1 - 1) * NE + i * kThreads)
                           : 0.f;
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int i = 0; i < EPT; ++i) val[i] = j0 + jj < p.S1 ? val[i] + l[jj][i] : val[i];
      }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = threadIdx.x + i * kThreads;
      int tok, ro;
      elem_coords<RB1>(e, &tok, &ro);
      const int n = row0 + ro;
      if (e >= NE || tok >= T || n >= p.r) continue;
      if (p.t32) p.t32[(int64_t)tok * p.ldt32 + n] = val[i];
      const uint32_t hi = f2bf(val[i]);
      const int64_t pi = tpack(tok, n, p.ldtb);
      store_coherent(p.thi + pi, (uint16_t)hi);
      if (SPLIT) store_coherent(p.tlo + pi, (uint16_t)f2bf(val[i] - bf2f(hi)));
    }
    wait_memory();  // this block's t is visible device-wide before it is counted
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = atomic_add_agent(p.ctl + CTL_TREADY, 1u);
      if (old == (uint32_t)(p.nb1 - 1)) {  // every row block has published
        store_relaxed(p.ctl + CTL_TREADY, 0u);
        if (p.wait) store_relaxed(p.ctl + CTL_GO, 1u);
      }
    }
    return;
  }

  int li = 0;  // the linear owning this stage-2 tile (workgroup-uniform)
  while (li + 1 < args.n && tile >= args.lin[li + 1].first2) ++li;
  const LinArgs& p = args.lin[li];
  if (RB2L != RB2 && p.rb2 == RB2L)
    stage2_tile<TB, RB2L, KSW2L, PFL, SPLIT, kBudget>(p, T, tile, red);
  else
    stage2_tile<TB, RB2, KSW2, PF, SPLIT, kBudget>(p, T, tile, red);
}

// t (fp32, caller's layout) -> fragment-packed bf16 (and bf16 residual) for a
// stage-2-only call.
__global__ __launch_bounds__(256) void split_t_kernel(const float* __restrict__ t, int64_t ldt,
                                                      int T, int N, uint16_t* thi, uint16_t* tlo,
                                                      int64_t ldtb) {
  const int64_t total = (int64_t)T * N;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int tok = (int)(e / N), n = (int)(e % N);
    const float v = t[(int64_t)tok * ldt + n];
    const uint32_t hi = f2bf(v);
    const int64_t pi = tpack(tok, n, ldtb);
    thi[pi] = (uint16_t)hi;
    if (tlo) tlo[pi] = (uint16_t)f2bf(v - bf2f(hi));
  }
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Tiling of one linear; identical on the sizing and launch sides.  Offsets
// are relative to the linear's data region (after the control blocks).
struct Plan {
  int TB, RB1, RB2, nb1, S1, kc1, n2;
  int64_t ldtb;
  size_t off_part, off_thi, off_tlo, bytes;
};

constexpr size_t kCtlBytes = (size_t)kMaxGroup * CTL_WORDS * 4;
// Stage-2 tiles a group must have at 64 rows each before it takes them (T > 32)
constexpr int kTallGroupTiles = 192;

Plan make_plan(int64_t T, int64_t d_in, int64_t r, int64_t d_out) {
  Plan pl{};
  pl.TB = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  pl.RB1 = pl.TB == 1 ? 1 : 2;
  // 64-row stage-2 tiles at T > 32 halve the re-reads of t (each tile reads
  // all of it) where there are tiles enough to fill the GPU anyway
  pl.RB2 = pl.TB == 4 && d_out >= 8192 ? 4 : 2;
  pl.nb1 = (int)((r + 16 * pl.RB1 - 1) / (16 * pl.RB1));
  pl.n2 = (int)((d_out + 16 * pl.RB2 - 1) / (16 * pl.RB2));
  // split K when a row block would hand one workgroup more than ~256 KiB
  // (128 KiB for 17..32 tokens) of weight and activation bytes: one
  // workgroup streams only ~40 GB/s.  Measured on the 7B shapes; more K
  // ranges than 6 cost more in meeting partials than they gain (32 tokens).
  const int64_t rows = 16 * pl.RB1 + std::min<int64_t>(T, 16 * pl.TB);
  const int64_t budget = pl.TB == 2 ? 131072 : 262144;
  const int64_t kc_max = std::max<int64_t>(32, (budget / (2 * rows)) / 32 * 32);
  const int64_t steps = (d_in + 31) / 32;
  pl.S1 = (int)((d_in + kc_max - 1) / kc_max);
  if (pl.TB == 2 && pl.S1 > 6) pl.S1 = 6;
  if (CTL_CNT + pl.nb1 > CTL_WORDS) pl.S1 = 1;  // no counters for that many row blocks
  pl.kc1 = (int)((steps + pl.S1 - 1) / pl.S1 * 32);
  if (pl.TB >= 2) pl.kc1 = (pl.kc1 + 63) / 64 * 64;  // ranges start on 128-byte lines
  pl.S1 = (int)((d_in + pl.kc1 - 1) / pl.kc1);
  pl.ldtb = (r + 31) / 32;  // t fragment-packed: k-steps per 16-token block
  const size_t nr1 = (size_t)pl.TB * pl.RB1 * 4 * 64;  // floats per stage-1 tile
  const size_t part = pl.S1 > 1 ? (size_t)pl.nb1 * pl.S1 * nr1 * 4 : 0;
  pl.off_part = 0;
  pl.off_thi = round_up(part, 256);
  const size_t tb_bytes = round_up((int64_t)pl.TB * pl.ldtb * 1024, 256);
  pl.off_tlo = pl.off_thi + tb_bytes;
  pl.bytes = pl.off_tlo + tb_bytes;
  return pl;
}

// Two builds per token block.  "spread": one workgroup per CU (the dynamic
// LDS is padded past half the CU's), up to 128 registers per lane, so a wave
// keeps a whole round of loads in flight -- for grids that fit the GPU at
// once (the dispatcher would otherwise stack two workgroups on one CU and
// halve the CUs streaming).  "dense": two workgroups per CU (64 registers,
// half-size rounds) for larger grids, which then keep all their stage-2 tiles
// resident.  Template arguments: weight rows per tile (16*RB1; 16*RB2, or
// 16*RB2L for linears the plan gives tall stage-2 tiles), k-steps per round
// (KSW1; KSW2, KSW2L), stage-2 prefetch depth (PF, PFL; multiples of the
// round).
constexpr int kLdsMax = 163840;

template <int TB, int RB1, int RB2, int RB2L, int KSW1, int KSW2, int KSW2L, int PF, int PFL,
          bool SPLIT, int WPC>
hipError_t launch_one(const DecArgs& a, int grid, hipStream_t st) {
  constexpr int budget = WPC == 1 ? kRedBudget1 : kRedBudget2;
  constexpr int NR1 = TB * RB1 * 4, NR2 = TB * (RB2L > RB2 ? RB2L : RB2) * 4;
  constexpr size_t red1 = (size_t)park_slots(NR1, budget) * NR1 * 256;
  constexpr size_t red2 = (size_t)park_slots(NR2, budget) * NR2 * 256;
  constexpr size_t red_bytes = red1 > red2 ? red1 : red2;
  static_assert(red_bytes <= (size_t)budget, "parked partials exceed the LDS budget");
  // stage-1 activation staging (T > 16): TB * 2 KiB per wave, inside the LDS
  constexpr size_t lds_min = WPC == 1 ? (size_t)kLdsMax / 2 + 1024 : 0;
  static_assert(TB < 2 || KSW1 % 2 != 0 ||
                    (red_bytes > lds_min ? red_bytes : lds_min) >= (size_t)kWaves * TB * 2048,
                "activation staging exceeds the dynamic LDS");
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(
            &decode_kernel<TB, RB1, RB2, RB2L, KSW1, KSW2, KSW2L, PF, PFL, SPLIT, WPC>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax - 1024);
  });
  const size_t lds = WPC == 1 ? std::max<size_t>(red_bytes, kLdsMax / 2 + 1024) : red_bytes;
  hipLaunchKernelGGL((decode_kernel<TB, RB1, RB2, RB2L, KSW1, KSW2, KSW2L, PF, PFL, SPLIT, WPC>),
                     dim3(grid),
                     dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int TB>
hipError_t launch_decode(const DecArgs& a, int grid, hipStream_t st) {
  const bool spread = grid <= 400;
  if (TB == 1)
    return spread ? launch_one<1, 1, 2, 2, 8, 4, 4, 4, 4, true, 1>(a, grid, st)
                  : launch_one<1, 1, 2, 2, 4, 2, 2, 2, 2, true, 2>(a, grid, st);
  if (TB == 2)
    return spread ? launch_one<2, 2, 2, 2, 4, 2, 2, 4, 4, false, 1>(a, grid, st)
                  : launch_one<2, 2, 2, 2, 2, 1, 1, 2, 2, false, 2>(a, grid, st);
  return launch_one<4, 2, 2, 4, 2, 2, 1, 4, 1, false, 1>(a, grid, st);
}

}  // namespace

size_t decode_group_workspace_bytes(const DecodeLinear* d, int n) {
  size_t bytes = kCtlBytes;
  for (int i = 0; i < n; ++i)
    bytes += round_up(make_plan(d[i].T, d[i].d_in, d[i].r, d[i].d_out).bytes, 256);
  return bytes;
}

size_t decode_workspace_bytes(int64_t T, int64_t d_in, int64_t r, int64_t d_out) {
  return kCtlBytes + round_up(make_plan(T, d_in, r, d_out).bytes, 256);
}

hipError_t decode_group_bf16(const DecodeLinear* ds, int n, hipStream_t st) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  const int64_t T = ds[0].T;
  char* ws = static_cast<char*>(ds[0].workspace);
  DecArgs a{};
  a.n = n;
  a.T = (int)T;
  size_t off = kCtlBytes;
  int n1 = 0, TB = 1;
  for (int i = 0; i < n; ++i) {
    const DecodeLinear& d = ds[i];
    const Plan pl = make_plan(T, d.d_in, d.r, d.d_out);
    TB = pl.TB;
    char* data = ws + off;
    off += round_up(pl.bytes, 256);
    LinArgs& L = a.lin[i];
    L.x = static_cast<const uint16_t*>(d.x);
    L.ldx = d.ldx;
    L.ut = static_cast<const uint16_t*>(d.Ut);
    L.ldu = d.ldu;
    L.vt = static_cast<const uint16_t*>(d.Vt);
    L.ldv = d.ldv;
    L.y = static_cast<uint16_t*>(d.y);
    L.ldy = d.ldy;
    L.yacc = d.y_acc;
    L.ldacc = d.ld_acc;
    L.t32 = d.t_io;
    L.ldt32 = d.ldt;
    L.thi = reinterpret_cast<uint16_t*>(data + pl.off_thi);
    L.tlo = reinterpret_cast<uint16_t*>(data + pl.off_tlo);
    L.ldtb = pl.ldtb;
    L.part = reinterpret_cast<float*>(data + pl.off_part);
    L.ctl = reinterpret_cast<uint32_t*>(ws + (size_t)i * CTL_WORDS * 4);
    L.d_in = (int)d.d_in;
    L.r = (int)d.r;
    L.d_out = (int)d.d_out;
    L.nb1 = pl.nb1;
    L.S1 = pl.S1;
    L.kc1 = pl.kc1;
    L.n2 = pl.n2;
    L.rb2 = pl.RB2;
    L.wait = 1;
    L.packed = d.packed ? 1 : 0;
    if (d.flags == 1) {  // stage 1 only
      L.n2 = 0;
      L.wait = 0;
    } else if (d.flags == 2) {  // stage 2 only: t from t_io
      const int64_t total = T * d.r;
      int blocks = (int)((total + 255) / 256);
      if (blocks > 1024) blocks = 1024;
      hipLaunchKernelGGL(split_t_kernel, dim3(blocks), dim3(256), 0, st, d.t_io, d.ldt, (int)T,
                         (int)d.r, L.thi, pl.TB == 1 ? L.tlo : (uint16_t*)nullptr, pl.ldtb);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      L.nb1 = 0;
      L.wait = 0;
    }
    L.first1 = n1;
    n1 += L.nb1 * L.S1;
  }
  // 64-row stage-2 tiles for a whole group at T > 32 when it still has tiles
  // enough to keep most CUs streaming V: on the 7B shapes at 64 tokens q,k,v
  // together (3 x 64 tiles) gain, o or down alone (64 tiles) lose.
  if (TB == 4) {
    int tall = 0;
    for (int i = 0; i < n; ++i)
      if (a.lin[i].n2) tall += (a.lin[i].d_out + 63) / 64;
    if (tall >= kTallGroupTiles)
      for (int i = 0; i < n; ++i)
        if (a.lin[i].n2) {
          a.lin[i].rb2 = 4;
          a.lin[i].n2 = (a.lin[i].d_out + 63) / 64;
        }
  }
  a.n1 = n1;
  int grid = n1;
  for (int i = 0; i < n; ++i) {
    a.lin[i].first2 = grid;
    grid += a.lin[i].n2;
  }
  if (grid == 0) return hipSuccess;
  switch (TB) {
    case 1: return launch_decode<1>(a, grid, st);
    case 2: return launch_decode<2>(a, grid, st);
    default: return launch_decode<4>(a, grid, st);
  }
}

hipError_t decode_linear_bf16(const DecodeLinear& d, hipStream_t st) {
  return decode_group_bf16(&d, 1, st);
}

}  // namespace lr
