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
// One kernel per launch, in one of two forms that share the tile code.  The
// persistent form (decode_pers_kernel, below; every launch it fits) holds
// one 8-wave workgroup per CU: workgroup w runs stage-1 tile w, then a run of
// stage-2 units, with the first V_r fragments issued before its wait for t.
// The tiled form (decode_kernel) lists every stage-1 tile and then every
// stage-2 tile of every linear of the launch, tile = blockIdx.x, two 8-wave
// workgroups per CU, so that while the stage-1 tiles stream U_r the stage-2
// tiles dispatched beside them already stream their first steps of V_r into
// registers and only then wait for t.  Workgroups are dispatched in index
// order and stage-1 tiles never wait, so a waiting stage-2 tile can never
// hold resources that a stage-1 tile it waits for still needs.
//   stage-1 tile: 16*RB1 rows of U_r^T over one of S1 K ranges.  S1 is chosen
//     per launch so that the launch has about one stage-1 tile per CU.  The 8
//     waves split the range into contiguous runs of k-steps and their partial
//     products meet in a fixed-order tree through LDS.  With S1 > 1 the
//     ranges of a row block meet in the workspace and the last to arrive sums
//     them in K-range order.  The finishing tile publishes its rows of t
//     (fp32 for t_io; bf16 for stage 2 in the fragment-packed layout the
//     weights use; for T <= 16 also the bf16 residual t - bf16(t), so stage 2
//     sees ~16 mantissa bits at the cost of a second MFMA) and counts itself;
//     the last row block raises the GO flag.
//   stage-2 tile: 16*RB2 rows of V_r^T over all of r.  Each wave issues the
//     loads of its first PF steps of V_r (for the 7B shapes, its whole run)
//     *before* waiting for GO, then reads t and finishes, writing y in bf16
//     (or adding into an fp32 accumulator).
// Synchronisation avoids cache-wide operations and hot addresses:
//   * data that crosses workgroups (partials, t) is written with
//     device-coherent stores and the writer waits for their completion before
//     it counts itself; partials are read back with device-coherent loads.
//     t is read with ordinary loads: no workgroup touches t's lines before
//     GO, and the kernel starts with the L2 invalidated, so no stale copy
//     can be hit;
//   * device-scope atomics on one address serialise (~10 ns each), so every
//     count is two-level: eight sub-counters (item index mod 8, each on a
//     256-byte line of its own) whose last arrivals count into a top counter.
// Counters live in the workspace and return to zero within the call: each
// counter is cleared by its own last arrival, and every workgroup counts its
// completion at its very end, the last one clearing GO (so GO is cleared
// after every stage-1 tile has set it and every stage-2 tile has passed its
// wait, even when a wait gave up).  Consecutive calls and graph replays need
// no memset.  Every wait is bounded: past the spin limit it records an error
// word (read and cleared by lowrank_workspace_check) and proceeds.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int kNW = 8;                      // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr uint32_t kOutside = 0x80000000u;  // past every buffer (tiles stay < 2 GiB)
constexpr int kCoherentLoad = 16;           // buffer-load cache policy: device scope
constexpr int kStreamLoad = 2;              // buffer-load cache policy: non-temporal
                                            // (weights, streamed once per call, should
                                            // not evict the activations and t)
constexpr int kMaxGroup = 8;                // linears per launch
constexpr int kRedBudget = 79 * 1024;       // LDS for parked partials: two workgroups per CU
constexpr int kStage1Tiles = 256;           // stage-1 tiles a launch aims at (one per CU)

std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};

// One control block (uint32 words) per linear of a launch, all of them at
// the start of the workspace.  Each hot word sits on a 256-byte line of its
// own.  Their place and size are the same for every call, so that data of
// one call never lands on words another call (of another shape or group
// size, same workspace) takes as zeroed counters.
enum {
  CTL_TSUB = 0,      // [8] stage-1 arrival sub-counters (row block mod 8)
  CTL_TTOP = 512,    // stage-1 arrival top counter
  CTL_GO = 576,      // t complete
  CTL_DSUB = 640,    // [8] completion sub-counters (workgroup index mod 8)
  CTL_DTOP = 1152,   // completion top counter
  CTL_ERR = kCtlErrWord,  // a wait gave up (kWaitErrorMagic)
  CTL_CNT = 1280,    // split-K arrival counters, one per stage-1 row block
  CTL_WORDS = kCtlBlockWords
};
constexpr int kSubStride = 64;  // words between sub-counters

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
  int first1, first2;  // index of the linear's first stage-1 / stage-2 tile
  int wait;          // stage-2 tiles wait for the stage-1 tiles of this launch
  int packed;        // weights fragment-packed
  int first_u, n2u;  // persistent form: first 16-row stage-2 unit, units
};

// A launch: up to kMaxGroup independent linears over the same T token rows;
// every stage-1 tile of every linear comes before every stage-2 tile.
struct DecArgs {
  LinArgs lin[kMaxGroup];
  int n, T, n1;  // linears, tokens, stage-1 tiles in all
  uint32_t spin_limit;
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

// Count one arrival of item idx of n items (n >= 1) into a two-level
// counter: sub-counter idx % 8, whose last arrival counts into the top one.
// Every counter is cleared by its own last arrival.  True for the arrival
// that completes the count.  Called by one thread.
__device__ __forceinline__ bool count_arrival(uint32_t* ctl, int sub_base, int top, int idx,
                                              int n) {
  const int j = idx & 7;
  const uint32_t nsub = (uint32_t)((n - j + 7) >> 3);  // items with index % 8 == j
  const uint32_t nused = (uint32_t)(n < 8 ? n : 8);
  uint32_t* s = ctl + sub_base + j * kSubStride;
  if (atomic_add_agent(s, 1u) != nsub - 1) return false;
  store_relaxed(s, 0u);
  if (atomic_add_agent(ctl + top, 1u) != nused - 1) return false;
  store_relaxed(ctl + top, 0u);
  return true;
}

// NB fragments of one k-step at byte offset step_off from the per-lane bases
// off[]; a dead step goes to an offset outside the buffer (reads zero, no
// memory access).
// POL: the loads' cache policy (kStreamLoad for weights, read once per call).
template <int NB, int POL = 0>
__device__ __forceinline__ void frag_load_at(u32x4 (&f)[NB], __amdgpu_buffer_rsrc_t rs,
                                             const uint32_t (&off)[NB], uint32_t step_off,
                                             bool live) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int o = (int)(live ? off[nb] + step_off : kOutside);
    f[nb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, POL));
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

// Wait until the linear's GO flag is up (one thread of the workgroup), at
// most spin_limit polls; past that, record the error word and go on.
__device__ __forceinline__ void wait_go(uint32_t* ctl, uint32_t spin_limit) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (load_relaxed(ctl + CTL_GO) == 0u) {
      if (spins++ >= spin_limit) {
        store_relaxed(ctl + CTL_ERR, kWaitErrorMagic);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// This wave's share of one tile: weight rows [row0, row0 + 16*RB) against
// A[0:T, kbeg:kend), over the wave's contiguous run of 32-wide k-steps.  Per
// round the wave issues the weight loads, then the activation loads, then
// the MFMAs.  Rows past T or N and steps past the wave's run fall outside
// the buffers and read zero, so the step loop has no branches; only a ragged
// last step (K range not a multiple of 32) is masked, after the loop.
// A stage-2 tile (WAIT) first issues the weight loads of its first PF steps,
// then waits for GO, then reads t.
// acc[tb][rb] lane l holds C[token tb*16 + 4*(l>>4) + v][row row0 + rb*16 + (l&15)].
template <int TB, int RB, int KSW, int PF, bool SPLIT, bool WAIT>
__device__ void tile_product(f32x4 (&acc)[TB][RB], const uint16_t* __restrict__ A,
                             const uint16_t* __restrict__ Alo, int64_t lda,
                             const uint16_t* __restrict__ B, int64_t ldb, bool packed, int T,
                             int N, int row0, int kbeg, int kend, uint32_t* ctl, bool wait,
                             uint32_t spin_limit, float* stage = nullptr) {
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
  const int per = XL ? 2 * ((nsteps + 2 * kNW - 1) / (2 * kNW))
                     : (nsteps + kNW - 1) / kNW;  // contiguous k-steps per wave
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
        frag_load_at<TB>(av[i], ra, aoff, (sb + i) * ASTEP, sb + i < s_full);
        if (SPLIT) frag_load_at<TB>(alv[i], ral, aoff, (sb + i) * ASTEP, sb + i < s_full);
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
      frag_load_at<RB, kStreamLoad>(bp[i], w.rs, w.off, (s_lo + i) * w.step, s_lo + i < s_full);
    if (wait) wait_go(ctl, spin_limit);
#pragma unroll
    for (int i0 = 0; i0 < PF; i0 += KSW) round(bp + i0, s_lo + i0);
    s0 = s_lo + PF;
  }
  for (; s0 < s_full; s0 += KSW) {
    u32x4 bv[KSW][RB];
#pragma unroll
    for (int i = 0; i < KSW; ++i)
      frag_load_at<RB, kStreamLoad>(bv[i], w.rs, w.off, (s0 + i) * w.step, s0 + i < s_full);
    round(bv, s0);
  }
  if (nfull < nsteps && nfull >= s_lo && nfull < s_hi) {
    // ragged last step of the K range, owned by this wave
    const int kk = nfull * 32 + kq;
    u32x4 bv[RB], av[TB], alv[TB];
    frag_load_at<RB, kStreamLoad>(bv, w.rs, w.off, nfull * w.step, true);
    frag_load_at<TB>(av, ra, aoff, nfull * ASTEP, true);
    if (SPLIT) frag_load_at<TB>(alv, ral, aoff, nfull * ASTEP, true);
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

// This wave's share of a stage-1 tile (persistent form) with every load of
// its run issued up front: the weight fragments of all its k-steps, then the
// activation fragments (for T > 16 as whole 128-byte lines, two k-steps per
// load, put through the wave's LDS slot as in tile_product), then the
// products.  A run longer than NS steps goes in chunks of NS.  Steps past the
// run read zero; a ragged last step of the K range comes after, masked.
template <int TB, int RB, int NS>
__device__ __forceinline__ void stage1_products(f32x4 (&acc)[TB][RB],
                                                const uint16_t* __restrict__ A, int64_t lda,
                                                const uint16_t* __restrict__ B, int64_t ldb,
                                                bool packed, int T, int N, int row0, int kbeg,
                                                int kend, float* stage) {
  constexpr bool XL = TB >= 2;
  static_assert(!XL || NS % 2 == 0, "whole pairs of steps");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = (lane >> 4) * 8;
  const int K = kend - kbeg;
  const WeightTile<RB> w(B, ldb, packed, N, row0, kbeg, kend, lane);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + kbeg, view_bytes(min(T, 16 * TB), K, lda));
  uint32_t aoff[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) aoff[tb] = (uint32_t)(((tb * 16 + (lane & 15)) * lda + kq) * 2);
  const int nsteps = (K + 31) / 32, nfull = K / 32;
  const int per = XL ? 2 * ((nsteps + 2 * kNW - 1) / (2 * kNW)) : (nsteps + kNW - 1) / kNW;
  const int s_lo = min(nsteps, wave * per);
  const int s_hi = min(nsteps, s_lo + per);
  const int s_full = min(s_hi, nfull);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[tb][r] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = s_lo; c0 < s_full; c0 += NS) {
    u32x4 wv[NS][RB];
#pragma unroll
    for (int i = 0; i < NS; ++i)
      frag_load_at<RB, kStreamLoad>(wv[i], w.rs, w.off, (c0 + i) * w.step, c0 + i < s_full);
    if constexpr (XL) {
      u32x4 ld[NS / 2][2 * TB];
#pragma unroll
      for (int pr = 0; pr < NS / 2; ++pr) {
        const int sp = c0 + 2 * pr;
#pragma unroll
        for (int q = 0; q < 2 * TB; ++q) {
          const int row = 8 * q + (lane >> 3), c = lane & 7;
          const bool live = sp + (c >> 2) < s_full;
          ld[pr][q] = bload(ra, live ? (uint32_t)((row * lda + sp * 32 + c * 8) * 2) : kOutside);
        }
      }
      uint8_t* xs = reinterpret_cast<uint8_t*>(stage) + wave * (TB * 2048);
#pragma unroll
      for (int pr = 0; pr < NS / 2; ++pr) {
        if (c0 + 2 * pr >= s_full) break;
#pragma unroll
        for (int q = 0; q < 2 * TB; ++q) {
          const int row = 8 * q + (lane >> 3), c = lane & 7;
          *reinterpret_cast<u32x4*>(xs + row * 128 + ((c ^ (row & 7)) << 4)) = ld[pr][q];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          u32x4 av[TB];
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            const int row = tb * 16 + (lane & 15), c = 4 * i + (lane >> 4);
            av[tb] = *reinterpret_cast<const u32x4*>(xs + row * 128 + ((c ^ (row & 7)) << 4));
          }
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < RB; ++r)
              acc[tb][r] = mfma16x16x32(av[tb], wv[2 * pr + i][r], acc[tb][r]);
        }
      }
    } else {
      u32x4 xa[NS][TB];
#pragma unroll
      for (int i = 0; i < NS; ++i) frag_load_at<TB>(xa[i], ra, aoff, (c0 + i) * 64, c0 + i < s_full);
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int r = 0; r < RB; ++r) acc[tb][r] = mfma16x16x32(xa[i][tb], wv[i][r], acc[tb][r]);
    }
  }
  if (nfull < nsteps && nfull >= s_lo && nfull < s_hi) {
    // ragged last step of the K range, owned by this wave
    const int kk = nfull * 32 + kq;
    u32x4 bv[RB], av[TB];
    frag_load_at<RB, kStreamLoad>(bv, w.rs, w.off, nfull * w.step, true);
    frag_load_at<TB>(av, ra, aoff, nfull * 64, true);
#pragma unroll
    for (int r = 0; r < RB; ++r) bv[r] = mask_tail_nb(bv[r], kk, K);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) av[tb] = mask_tail_nb(av[tb], kk, K);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[tb][r] = mfma16x16x32(av[tb], bv[r], acc[tb][r]);
  }
}

// LDS slots for parking a tile of NR accumulator registers per lane: one
// per wave when kNW x NR x 256 bytes fit the budget, else kNW/2 (waves w and
// w + kNW/2 added in registers first).
constexpr int park_slots(int NR, int lds_budget) {
  return kNW * NR * 256 <= lds_budget ? kNW : kNW / 2;
}

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

// Park the waves' partial products in NSLOT slots whose sum is the tile.
template <int TB, int RB, int NSLOT>
__device__ __forceinline__ void park(f32x4 (&acc)[TB][RB], float* red) {
  const int wave = threadIdx.x >> 6;
  constexpr int H = kNW / 2;
  if (NSLOT == kNW) {
    park_slot<TB, RB>(acc, red, wave);
    lds_barrier();
    return;
  }
  constexpr int NR = TB * RB * 4;
  if (wave >= H) park_slot<TB, RB>(acc, red, wave - H);
  lds_barrier();
  if (wave < H) {
    const float* b = red + wave * NR * 64 + (threadIdx.x & 63);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[tb][r][v] += b[((tb * RB + r) * 4 + v) * 64];
  }
  lds_barrier();
  if (wave < H) park_slot<TB, RB>(acc, red, wave);
  lds_barrier();
}

// Element e of a parked tile summed over the slots, pairwise in a fixed order
// (slot w + kNW/2 -- already added in registers when there are kNW/2 slots --
// then + kNW/4, ..., + 1: the same order either way).
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

// The workgroup's completion: every tile of a waiting linear counts itself
// at its very end; the last one clears GO for the next call.
__device__ __forceinline__ void count_done(const LinArgs& p, int idx) {
  if (p.wait && threadIdx.x == 0 &&
      count_arrival(p.ctl, CTL_DSUB, CTL_DTOP, idx, p.nb1 * p.S1 + p.n2))
    store_relaxed(p.ctl + CTL_GO, 0u);
}

struct NoHook {
  __device__ __forceinline__ void others() const {}
  __device__ __forceinline__ void first() const {}
};

// One stage-1 tile: 16*RB1 rows of U_r^T over one K range, then (for the last
// K range of the row block to arrive) t published and counted.  COUNT: the
// tile counts its own completion.  The hook lets the persistent form issue
// its first V_r loads as early as the counters allow: a wave's counter
// (vmcnt) covers its loads and stores alike, in issue order, so a wave must
// not have loads in flight when it waits for its own stores or for an
// atomic's result.  hook.others() runs on every wave once its stores are
// complete and nothing of the tile is left to load (waves 1..7 issue there),
// hook.first() once thread 0's counting atomics have returned (wave 0).
template <int TB, int RB1, int KSW1, bool COUNT = true, class Hook = NoHook, int NS1 = 0>
__device__ __forceinline__ void stage1_tile(const LinArgs& p, int T, int t1, float* red,
                                            const Hook& hook = Hook()) {
  __shared__ uint32_t sh_last;
  constexpr int NR = TB * RB1 * 4, NE = NR * 64;
  constexpr int EPT = (NE + kThreads - 1) / kThreads;  // elements per thread
  const int blk = t1 / p.S1, s = t1 % p.S1;
  const int row0 = blk * 16 * RB1;
  const int kbeg = s * p.kc1, kend = min(p.d_in, kbeg + p.kc1);
  f32x4 acc[TB][RB1];
  if constexpr (NS1 > 0)
    stage1_products<TB, RB1, NS1>(acc, p.x, p.ldx, p.ut, p.ldu, p.packed != 0, T, p.r, row0,
                                  kbeg, kend, red);
  else
    tile_product<TB, RB1, KSW1, KSW1, false, false>(acc, p.x, nullptr, p.ldx, p.ut, p.ldu,
                                                    p.packed != 0, T, p.r, row0, kbeg, kend,
                                                    p.ctl, false, 0u, red);
  constexpr int NS = park_slots(NR, kRedBudget);
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
    lds_barrier();  // every wave's partials are complete
    if (threadIdx.x == 0) {
      const uint32_t old = atomic_add_agent(p.ctl + CTL_CNT + blk, 1u);
      sh_last = old == (uint32_t)(p.S1 - 1);
      if (sh_last) store_relaxed(p.ctl + CTL_CNT + blk, 0u);  // every sibling has arrived
    }
    lds_barrier();
    if (!sh_last) {
      hook.others();
      hook.first();
      if (COUNT) count_done(p, t1);
      return;
    }
    constexpr int JB = 4;
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
  const bool split = TB == 1;
  // the bf16 operand only for a stage 2 in this launch (a stage-1-only
  // linear's t leaves as fp32 t_io, which the end of the kernel publishes)
  const bool pub = p.wait != 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = threadIdx.x + i * kThreads;
    int tok, ro;
    elem_coords<RB1>(e, &tok, &ro);
    const int n = row0 + ro;
    if (e >= NE || tok >= T || n >= p.r) continue;
    if (p.t32) p.t32[(int64_t)tok * p.ldt32 + n] = val[i];
    if (!pub) continue;
    const uint32_t hi = f2bf(val[i]);
    const int64_t pi = tpack(tok, n, p.ldtb);
    store_coherent(p.thi + pi, (uint16_t)hi);
    if (split) store_coherent(p.tlo + pi, (uint16_t)f2bf(val[i] - bf2f(hi)));
  }
  if (pub) wait_memory();  // this block's t is visible device-wide before it is counted
  hook.others();
  lds_barrier();  // every wave's t is complete
  if (p.wait && threadIdx.x == 0 && count_arrival(p.ctl, CTL_TSUB, CTL_TTOP, blk, p.nb1))
    store_relaxed(p.ctl + CTL_GO, 1u);
  hook.first();
  if (COUNT) count_done(p, t1);
}

// One stage-2 tile: 16*RB2 rows of V_r^T over all of r, then y.
template <int TB, int RB2, int KSW2, int PF, bool SPLIT>
__device__ __forceinline__ void stage2_tile(const LinArgs& p, int T, int t2, float* red,
                                            uint32_t spin_limit) {
  constexpr int NR = TB * RB2 * 4, NE = NR * 64;
  constexpr int EPT = (NE + kThreads - 1) / kThreads;
  const int row0 = t2 * 16 * RB2;
  f32x4 acc[TB][RB2];
  tile_product<TB, RB2, KSW2, PF, SPLIT, true>(acc, p.thi, p.tlo, p.ldtb, p.vt, p.ldv,
                                               p.packed != 0, T, p.d_out, row0, 0, p.r,
                                               p.ctl, p.wait != 0, spin_limit);
  constexpr int NS = park_slots(NR, kRedBudget);
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
  count_done(p, p.nb1 * p.S1 + t2);
}

template <int TB, int RB1, int RB2, int KSW1, int KSW2, int PF, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void decode_kernel(DecArgs args) {
  extern __shared__ __attribute__((aligned(16))) float red[];  // [slots][NR][64]
  const int tile = (int)blockIdx.x;
  const int T = args.T;
  if (tile < args.n1) {
    int li = 0;  // the linear owning this stage-1 tile (workgroup-uniform)
    while (li + 1 < args.n && tile >= args.lin[li + 1].first1) ++li;
    stage1_tile<TB, RB1, KSW1>(args.lin[li], T, tile - args.lin[li].first1, red);
    return;
  }
  int li = 0;  // the linear owning this stage-2 tile (workgroup-uniform)
  while (li + 1 < args.n && tile >= args.lin[li + 1].first2) ++li;
  stage2_tile<TB, RB2, KSW2, PF, SPLIT>(args.lin[li], T, tile - args.lin[li].first2, red,
                                        args.spin_limit);
}


// ------------------------------------------------------------ persistent form
// One workgroup per CU (8 waves, up to 256 registers each), G = the CU count,
// all resident at once.  Workgroup w first runs stage-1 tile w (w < n1), then
// its share of stage-2 units: units are 16 rows of one linear's V_r^T over all
// of r, listed linear by linear, and each workgroup takes a contiguous run of
// them sized so that every workgroup streams about the same bytes of U_r and
// V_r in all.  Wave i takes k-steps [i*per, (i+1)*per) of every unit (per =
// ceil(steps / 8) <= PER): it loads its slice of t once per linear and keeps
// the V_r fragments of its next D units in flight in registers, the first of
// them issued before the wait for GO (for a stage-1 workgroup, as soon as its
// own products are done), so each CU streams without a gap across the
// hand-over.  Per unit the 8 waves' partial products meet in LDS (two
// buffers, one barrier per unit) and the sum in a fixed order gives y.
// Every workgroup counts its completion once; the last clears every GO.
constexpr int kMaxWG = 256;
constexpr int kPersLds = 96 * 1024;  // over half a CU: one workgroup per CU
constexpr int kPreUnits = 2;         // ring slots in flight across the wait for GO

struct PersArgs {
  LinArgs lin[kMaxGroup];
  int n, T, n1, G;
  uint32_t spin_limit;
  int pre;  // ring slots a stage-1 workgroup issues before its t is published
            // (the others issue them all: they have nothing else to stream)
  int u_beg[kMaxWG + 1];  // stage-2 units of workgroup w: [u_beg[w], u_beg[w + 1])
};

__device__ __forceinline__ int linear_of_unit(const PersArgs& a, int u) {
  int li = 0;
  while (li + 1 < a.n && u >= a.lin[li + 1].first_u) ++li;
  return li;
}

// GO of one linear (thread 0 polls, at most spin_limit times), then a
// barrier that does not wait for this wave's loads in flight.
__device__ __forceinline__ void wait_go_light(uint32_t* ctl, uint32_t spin_limit) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (load_relaxed(ctl + CTL_GO) == 0u) {
      if (spins++ >= spin_limit) {
        store_relaxed(ctl + CTL_ERR, kWaitErrorMagic);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  lds_barrier();
}

// Where this wave's fragments of one stage-2 unit come from.
struct UnitSrc {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off, step;
  int dead;  // leading slots with no step (PER - s_n)
};

template <int TB, int PER, int D, bool SPLIT>
struct Stage2 {
  u32x4 ring[D][PER];  // V_r fragments of the next D units, this wave's k-steps
  int ub, ue;          // the workgroup's units
  int pre;             // ring slots issued by prefetch()

  // This wave's k-steps of linear p are [s_hi - s_n, s_hi), s_n <= PER,
  // held right-aligned in PER slots: slot i is step s_hi - PER + i, live for
  // i >= PER - s_n.  The ragged last step of r (r % 32 != 0) can only be
  // the last wave's last step, so it always sits in slot PER - 1.
  __device__ __forceinline__ static void wave_steps(const LinArgs& p, int* s_hi, int* s_n) {
    const int nsteps = (p.r + 31) / 32, per = (nsteps + kNW - 1) / kNW;
    // wave-uniform (the buffer resources built from it must be scalar)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lo = min(nsteps, wave * per);
    *s_hi = min(nsteps, lo + per);
    *s_n = *s_hi - lo;
  }

  __device__ __forceinline__ static UnitSrc locate(const PersArgs& a, int u) {
    const int lane = threadIdx.x & 63;
    const LinArgs& p = a.lin[linear_of_unit(a, u)];
    const int b = u - p.first_u;
    int s_hi, s_n;
    wave_steps(p, &s_hi, &s_n);
    const int s0 = s_hi - s_n;  // first live step (slot PER - s_n)
    UnitSrc src;
    if (p.packed) {
      src.rs = make_rsrc(p.vt + ((int64_t)b * p.ldv + s0) * 512, (uint64_t)s_n * 1024);
      src.off = lane * 16;
      src.step = 1024;
    } else {
      src.rs = make_rsrc(p.vt + (int64_t)b * 16 * p.ldv + s0 * 32,
                         view_bytes(min(16, p.d_out - b * 16), p.r - s0 * 32, p.ldv));
      src.off = (uint32_t)(((lane & 15) * p.ldv + (lane >> 4) * 8) * 2);
      src.step = 64;
    }
    src.dead = PER - s_n;
    return src;
  }

  __device__ __forceinline__ void issue_frag(int slot, int i, const UnitSrc& src) {
    const int j = i - src.dead;  // live step index within the run
    ring[slot][i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   src.rs, (int)(j >= 0 ? src.off + (uint32_t)j * src.step : kOutside), 0,
                   kStreamLoad));
  }

  __device__ __forceinline__ void issue(const PersArgs& a, int slot, int u) {
    const UnitSrc src = locate(a, u);
#pragma unroll
    for (int i = 0; i < PER; ++i) issue_frag(slot, i, src);
  }

  // The first `pre` units, before the wait for GO.  Only about as many bytes
  // as cover the hand-over: more would queue in memory ahead of the other
  // workgroups' t stores and counter atomics and delay GO itself.
  __device__ __forceinline__ void prefetch(const PersArgs& a, int n) {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < n && ub + d < ue) issue(a, d, ub + d);
  }

  // t slice of linear p (after its GO): th[i][tb] the fragment of slot i's
  // step and token block tb; lanes of tokens >= T and dead slots read zero;
  // the ragged step's elements past r masked.
  __device__ __forceinline__ static void load_t(const LinArgs& p, int T, u32x4 (&th)[PER][TB],
                                                u32x4 (&tl)[PER][TB]) {
    const int lane = threadIdx.x & 63;
    int s_hi, s_n;
    wave_steps(p, &s_hi, &s_n);
    const uint64_t bytes = (uint64_t)TB * p.ldtb * 1024;
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(p.thi, bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(SPLIT ? p.tlo : p.thi, bytes);
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int sidx = s_hi - PER + i;
        const bool live = i >= PER - s_n && tb * 16 + (lane & 15) < T;
        const uint32_t o = live ? (uint32_t)(((tb * p.ldtb + sidx) * 64 + lane) * 16) : kOutside;
        th[i][tb] = bload(rh, o);
        if (SPLIT) tl[i][tb] = bload(rl, o);
      }
    if (s_hi * 32 > p.r) {  // this wave holds the ragged step, in slot PER - 1
      const int k0 = (s_hi - 1) * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        th[PER - 1][tb] = mask_tail_nb(th[PER - 1][tb], k0, p.r);
        if (SPLIT) tl[PER - 1][tb] = mask_tail_nb(tl[PER - 1][tb], k0, p.r);
      }
    }
  }

  // Every unit of the workgroup (after prefetch()).  Each consumed fragment
  // is replaced at once by the same fragment of the unit D ahead, so a wave
  // keeps D * PER fragments in flight without bursts.
  __device__ __forceinline__ void run(const PersArgs& a, float* red) {
    const int T = a.T;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int NR = TB * 4, NE = NR * 64;
    u32x4 th[PER][TB], tl[PER][TB];
    int cur = -1, rag_k0 = 0;
    bool rag = false;
    if (ub >= ue) return;
    // t of the first linear, then the ring slots not yet in flight (issued
    // after the t loads, so that waiting for t does not wait for them)
    {
      const int li = linear_of_unit(a, ub);
      const LinArgs& p = a.lin[li];
      load_t(p, T, th, tl);
      int s_hi, s_n;
      wave_steps(p, &s_hi, &s_n);
      rag = s_hi * 32 > p.r;
      rag_k0 = (s_hi - 1) * 32 + (lane >> 4) * 8;
      cur = li;
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d >= pre && ub + d < ue) issue(a, d, ub + d);
    for (int u0 = ub; u0 < ue; u0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int u = u0 + d;
        if (u >= ue) break;
        const int li = linear_of_unit(a, u);
        const LinArgs& p = a.lin[li];
        if (li != cur) {
          load_t(p, T, th, tl);
          int s_hi, s_n;
          wave_steps(p, &s_hi, &s_n);
          rag = s_hi * 32 > p.r;
          rag_k0 = (s_hi - 1) * 32 + (lane >> 4) * 8;
          cur = li;
        }
        const bool more = u + D < ue;
        UnitSrc nx;
        if (more) nx = locate(a, u + D);
        // the ragged step's V_r elements past r may hold anything (NaN)
        if (rag) ring[d][PER - 1] = mask_tail_nb(ring[d][PER - 1], rag_k0, p.r);
        f32x4 acc[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < PER; ++i) {
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            acc[tb] = mfma16x16x32(th[i][tb], ring[d][i], acc[tb]);
            if (SPLIT) acc[tb] = mfma16x16x32(tl[i][tb], ring[d][i], acc[tb]);
          }
          if (more) issue_frag(d, i, nx);  // refill the fragment just consumed
        }
        // the waves' partial products meet in LDS buffer (u - ub) & 1
        float* buf = red + ((u - ub) & 1) * kNW * NE;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int v = 0; v < 4; ++v) buf[wave * NE + (tb * 4 + v) * 64 + lane] = acc[tb][v];
        lds_barrier();
        const int b = u - p.first_u;
        for (int e = threadIdx.x; e < NE; e += kThreads) {
          float s8[kNW];
#pragma unroll
          for (int w = 0; w < kNW; ++w) s8[w] = buf[w * NE + e];
#pragma unroll
          for (int h = kNW / 2; h >= 1; h >>= 1)
#pragma unroll
            for (int w = 0; w < h; ++w) s8[w] += s8[w + h];
          int tok, ro;
          elem_coords<1>(e, &tok, &ro);
          const int n = b * 16 + ro;
          if (tok >= T || n >= p.d_out) continue;
          if (p.yacc)
            p.yacc[(int64_t)tok * p.ldacc + n] += s8[0];
          else
            p.y[(int64_t)tok * p.ldy + n] = (uint16_t)f2bf(s8[0]);
        }
      }
    }
  }
};

// Issue the persistent form's first V_r loads from inside a stage-1 tile.
template <class S2>
struct PrefetchHook {
  S2* s2;
  const PersArgs* a;
  __device__ __forceinline__ void others() const {
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) != 0) s2->prefetch(*a, a->pre);
  }
  __device__ __forceinline__ void first() const {
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) s2->prefetch(*a, a->pre);
  }
};

template <int TB, int RB1, int KSW1, int PER, int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_pers_kernel(PersArgs args) {
  extern __shared__ __attribute__((aligned(16))) float red[];
  // the arguments read in place from the kernel-argument segment (a
  // reference to the by-value parameter makes the compiler copy all 2.6 KB
  // of it to scratch memory once indices into it are not constants)
  (void)args;
  const PersArgs& a = *(const PersArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int w = (int)blockIdx.x;
  using S2 = Stage2<TB, PER, D, SPLIT>;
  S2 s2;
  s2.ub = a.u_beg[w];
  s2.ue = a.u_beg[w + 1];
  s2.pre = w < a.n1 ? a.pre : D;
  if (w < a.n1) {
    int li = 0;  // the linear owning this stage-1 tile (workgroup-uniform)
    while (li + 1 < a.n && w >= a.lin[li + 1].first1) ++li;
    const PrefetchHook<S2> hook{&s2, &a};
    // k-steps of a wave's stage-1 run loaded at once
    constexpr int NS1 = TB == 1 ? 8 : (TB == 2 ? 8 : 8);
    stage1_tile<TB, RB1, KSW1, false, PrefetchHook<S2>, NS1>(a.lin[li], a.T,
                                                             w - a.lin[li].first1, red, hook);
  } else {
    s2.prefetch(a, D);
  }
  // wait for t of every linear the units belong to, then count this
  // workgroup past its waits; the last one clears every GO
  if (s2.ub < s2.ue) {
    const int l0 = linear_of_unit(a, s2.ub), l1 = linear_of_unit(a, s2.ue - 1);
    for (int li = l0; li <= l1; ++li)
      if (a.lin[li].wait && a.lin[li].n2u) wait_go_light(a.lin[li].ctl, a.spin_limit);
  }
  // (a launch where no linear waits -- stage 1 only -- has nothing to clear)
  bool waits = false;
  for (int li = 0; li < a.n; ++li) waits = waits || a.lin[li].wait;
  if (waits && threadIdx.x == 0 && count_arrival(a.lin[0].ctl, CTL_DSUB, CTL_DTOP, w, a.G))
    for (int li = 0; li < a.n; ++li)
      if (a.lin[li].wait) store_relaxed(a.lin[li].ctl + CTL_GO, 0u);
  s2.run(a, red);
}

// t (fp32, caller's layout) -> fragment-packed bf16 (and bf16 residual) for a
// stage-2-only call.
// Stage-2-only members of a launch: their caller's fp32 t re-laid into the
// fragment-packed bf16 operand (plus the bf16 residual for T <= 16), all
// members in one launch (blockIdx.y = member).
struct SplitT {
  const float* t;
  int64_t ldt;
  int N;
  uint16_t* thi;
  uint16_t* tlo;
  int64_t ldtb;
};
struct SplitArgs {
  SplitT m[kMaxGroup];
  int T;
};

__global__ __launch_bounds__(256) void split_t_kernel(SplitArgs a) {
  const SplitT& s = a.m[blockIdx.y];
  const int64_t total = (int64_t)a.T * s.N;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int tok = (int)(e / s.N), n = (int)(e % s.N);
    const float v = s.t[(int64_t)tok * s.ldt + n];
    const uint32_t hi = f2bf(v);
    const int64_t pi = tpack(tok, n, s.ldtb);
    s.thi[pi] = (uint16_t)hi;
    if (s.tlo) s.tlo[pi] = (uint16_t)f2bf(v - bf2f(hi));
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

int token_blocks(int64_t T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }
int stage1_rows(int TB) { return TB == 1 ? 1 : 2; }  // RB1

// K ranges per stage-1 row block for a launch whose linears have nb_total
// row blocks in all: about one stage-1 tile per CU, at most 8 ranges, each
// at least 512 deep.
int stage1_ranges(int64_t nb_total, int64_t d_in) {
  int64_t s = nb_total > 0 ? kStage1Tiles / nb_total : 1;
  s = std::min<int64_t>(s, std::max<int64_t>(1, d_in / 512));
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, 8));
}

Plan make_plan(int64_t T, int64_t d_in, int64_t r, int64_t d_out, int S1) {
  Plan pl{};
  pl.TB = token_blocks(T);
  pl.RB1 = stage1_rows(pl.TB);
  pl.RB2 = 2;
  pl.nb1 = (int)((r + 16 * pl.RB1 - 1) / (16 * pl.RB1));
  pl.n2 = (int)((d_out + 16 * pl.RB2 - 1) / (16 * pl.RB2));
  const int64_t steps = (d_in + 31) / 32;
  pl.S1 = std::max(1, S1);
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

// The K-range count of a launch (identical on the sizing and launch sides):
// from the row blocks of the linears that run stage 1.
int group_ranges(const DecodeLinear* ds, int n) {
  const int64_t T = ds[0].T;
  const int RB1 = stage1_rows(token_blocks(T));
  int64_t nb = 0, din = INT64_MAX;
  for (int i = 0; i < n; ++i) {
    if (ds[i].flags == 2) continue;  // stage 2 only
    nb += (ds[i].r + 16 * RB1 - 1) / (16 * RB1);
    din = std::min(din, ds[i].d_in);
  }
  return nb ? stage1_ranges(nb, din) : 1;
}

constexpr int kLdsMax = 163840;

template <int TB, int RB1, int RB2, int KSW1, int KSW2, int PF, bool SPLIT>
hipError_t launch_one(const DecArgs& a, int grid, hipStream_t st) {
  constexpr int NR1 = TB * RB1 * 4, NR2 = TB * RB2 * 4;
  constexpr size_t red1 = (size_t)park_slots(NR1, kRedBudget) * NR1 * 256;
  constexpr size_t red2 = (size_t)park_slots(NR2, kRedBudget) * NR2 * 256;
  constexpr size_t stage_bytes = (TB >= 2 && KSW1 % 2 == 0) ? (size_t)kNW * TB * 2048 : 0;
  constexpr size_t lds = std::max(std::max(red1, red2), stage_bytes);
  static_assert(lds <= (size_t)kRedBudget, "LDS exceeds half a CU");
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<TB, RB1, RB2, KSW1, KSW2, PF, SPLIT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax / 2);
  });
  hipLaunchKernelGGL((decode_kernel<TB, RB1, RB2, KSW1, KSW2, PF, SPLIT>), dim3(grid),
                     dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int TB>
hipError_t launch_decode(const DecArgs& a, int grid, bool thin, hipStream_t st) {
  // <TB, RB1, RB2, KSW1, KSW2, PF, SPLIT>: PF covers a wave's whole run of
  // V_r for r up to 8 * 8 * 32 = 2048 (6 * 8 * 32 at 64 tokens).  thin:
  // 16-row stage-2 tiles (launches with few output rows)
  if (TB == 1)
    return thin ? launch_one<1, 1, 1, 8, 4, 8, true>(a, grid, st)
                : launch_one<1, 1, 2, 8, 4, 8, true>(a, grid, st);
  if (TB == 2)
    return thin ? launch_one<2, 2, 1, 4, 2, 8, false>(a, grid, st)
                : launch_one<2, 2, 2, 4, 2, 8, false>(a, grid, st);
  return launch_one<4, 2, 2, 2, 2, 6, false>(a, grid, st);
}

// Registers of the persistent form: t slice PER x TB (x2 for the bf16
// residual), accumulators TB x 4, and D ring slots of PER fragments each,
// within ~220 of the 256 a wave may hold (208 with the bf16 residual).
// Ring slots of the persistent form: about kRingFrags fragments (1 KiB
// each) in flight per wave, 64 KiB per CU -- enough to keep HBM busy at this
// part's latency, few enough that no workgroup's loads queue far ahead of
// the others' -- within the registers left by the t slice (PER x TB, twice
// with the bf16 residual) and the accumulators.
#ifndef LR_RING_FRAGS
#define LR_RING_FRAGS 8
#endif
constexpr int kRingFrags = LR_RING_FRAGS;
constexpr int ring_depth(int TB, int PER, bool split) {
  const int t = PER * TB * 4 * (split ? 2 : 1) + TB * 4;
  const int fit = ((split ? 208 : 220) - t) / (PER * 4);
  const int want = (kRingFrags + PER - 1) / PER;
  const int d = want < fit ? want : fit;
  return d < 1 ? 1 : d;
}

template <int TB, int PER>
hipError_t launch_pers_one(const PersArgs& a, hipStream_t st) {
  constexpr bool SPLIT = TB == 1;
  constexpr int RB1 = TB == 1 ? 1 : 2, KSW1 = TB == 1 ? 8 : (TB == 2 ? 4 : 2);
  constexpr int D = ring_depth(TB, PER, SPLIT);
  constexpr int NR1 = TB * RB1 * 4;
  constexpr size_t park1 = (size_t)park_slots(NR1, kRedBudget) * NR1 * 256;
  constexpr size_t stage_bytes = (TB >= 2 && KSW1 % 2 == 0) ? (size_t)kNW * TB * 2048 : 0;
  constexpr size_t red2 = (size_t)2 * kNW * TB * 4 * 64 * 4;
  static_assert(park1 <= (size_t)kPersLds && stage_bytes <= (size_t)kPersLds &&
                    red2 <= (size_t)kPersLds,
                "LDS of the persistent form");
  auto* fn = &decode_pers_kernel<TB, RB1, KSW1, PER, D, SPLIT>;
  static std::once_flag once;
  std::call_once(once, [fn] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kPersLds);
  });
  hipLaunchKernelGGL(fn, dim3(a.G), dim3(kThreads), kPersLds, st, a);
  return hipGetLastError();
}

// PER the persistent form instantiates for a run of per k-steps per wave.
int per_class(int per) { return per <= 2 ? 2 : (per <= 4 ? 4 : (per <= 6 ? 6 : 8)); }

template <int TB>
hipError_t launch_pers(const PersArgs& a, int per, hipStream_t st) {
  switch (per_class(per)) {
    case 2: return launch_pers_one<TB, 2>(a, st);
    case 4: return launch_pers_one<TB, 4>(a, st);
    case 6: return launch_pers_one<TB, 6>(a, st);
    default: return launch_pers_one<TB, 8>(a, st);
  }
}

// CUs of the current device (cached per device).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cache[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = 0;
    cache[dev] = v;
  }
  return cache[dev];
}

// The persistent form of a launch whose tiling is in d (stage-1 tiles
// first1/nb1/S1, stage-2 linears): G workgroups, each a contiguous run of
// stage-2 units.  Every workgroup streams V_r at about the same rate once GO
// is up; before it, a stage-1 workgroup streams its U_r tile and `pre` units
// of V_r, the others D units of V_r.  So the others take D - pre units more
// and the V_r bytes after GO even out.  False when the launch does not fit
// the form (a rank over 2048, more stage-1 tiles than CUs); the tiled form
// then runs.
bool plan_persistent(const DecArgs& d, int TB, PersArgs* a, int* per_out) {
  const int cus = std::min(device_cus(), kMaxWG);
  if (cus <= 0 || d.n1 > cus) return false;
  int per = 1, units = 0;
  double v_bytes = 0;
  for (int i = 0; i < d.n; ++i) {
    const LinArgs& L = d.lin[i];
    const int nsteps = (L.r + 31) / 32;
    if (L.n2) per = std::max(per, (nsteps + kNW - 1) / kNW);
    v_bytes += (double)(L.n2 ? (L.d_out + 15) / 16 : 0) * nsteps * 1024;
    units += L.n2 ? (L.d_out + 15) / 16 : 0;
  }
  if (per > 8) return false;
  const int G = std::max(1, std::min(cus, std::max(d.n1, units)));
  a->n = d.n;
  a->T = d.T;
  a->n1 = d.n1;
  a->G = G;
  a->spin_limit = d.spin_limit;
  a->pre = kPreUnits;
  int u = 0;
  for (int i = 0; i < d.n; ++i) {
    a->lin[i] = d.lin[i];
    a->lin[i].first_u = u;
    a->lin[i].n2u = d.lin[i].n2 ? (d.lin[i].d_out + 15) / 16 : 0;
    u += a->lin[i].n2u;
  }
  const int D = ring_depth(TB, per_class(per), TB == 1);
  const double unit = units ? v_bytes / units : 0;
  double extra = std::max(0, D - a->pre) * unit;
  const int others = G - std::min(G, d.n1);
  double base = (v_bytes - others * extra) / G;
  if (base < 0) {
    base = 0;
    extra = others ? v_bytes / others : 0;
  }
  double want = 0, vcum = 0;
  int next = 0;
  a->u_beg[0] = 0;
  for (int w = 0; w < G; ++w) {
    want += base + (w >= d.n1 ? extra : 0);
    while (next < units) {
      int lj = 0;
      while (lj + 1 < d.n && next >= a->lin[lj + 1].first_u) ++lj;
      const double ub = (double)((a->lin[lj].r + 31) / 32) * 1024;
      if (vcum + 0.5 * ub > want) break;
      vcum += ub;
      ++next;
    }
    a->u_beg[w + 1] = w + 1 == G ? units : next;
  }
  *per_out = per;
  return true;
}

}  // namespace

void set_spin_limit(uint32_t polls) { g_spin_limit.store(polls); }

size_t decode_group_workspace_bytes(const DecodeLinear* d, int n) {
  size_t bytes = kCtlBytes;
  const int S1 = group_ranges(d, n);
  for (int i = 0; i < n; ++i)
    bytes += round_up(make_plan(d[i].T, d[i].d_in, d[i].r, d[i].d_out, S1).bytes, 256);
  return bytes;
}

size_t decode_workspace_bytes(int64_t T, int64_t d_in, int64_t r, int64_t d_out) {
  DecodeLinear d{T, d_in, r, d_out};
  return decode_group_workspace_bytes(&d, 1);
}

hipError_t decode_group_bf16(const DecodeLinear* ds, int n, hipStream_t st) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  const int64_t T = ds[0].T;
  char* ws = static_cast<char*>(ds[0].workspace);
  DecArgs a{};
  a.n = n;
  a.T = (int)T;
  a.spin_limit = g_spin_limit.load();
  const int S1 = group_ranges(ds, n);
  size_t off = kCtlBytes;
  int n1 = 0, TB = 1;
  SplitArgs sa{};
  sa.T = (int)T;
  int nsplit = 0;
  int64_t split_el = 0;
  for (int i = 0; i < n; ++i) {
    const DecodeLinear& d = ds[i];
    const Plan pl = make_plan(T, d.d_in, d.r, d.d_out, S1);
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
    L.wait = 1;
    L.packed = d.packed ? 1 : 0;
    if (d.flags == 1) {  // stage 1 only
      L.n2 = 0;
      L.wait = 0;
    } else if (d.flags == 2) {  // stage 2 only: t from t_io
      sa.m[nsplit++] = SplitT{d.t_io, d.ldt, (int)d.r, L.thi,
                              pl.TB == 1 ? L.tlo : (uint16_t*)nullptr, pl.ldtb};
      split_el = std::max(split_el, T * d.r);
      L.nb1 = 0;
      L.wait = 0;
    }
    L.first1 = n1;
    n1 += L.nb1 * L.S1;
  }
  if (nsplit) {
    const int blocks = (int)std::min<int64_t>((split_el + 255) / 256, 1024);
    hipLaunchKernelGGL(split_t_kernel, dim3(blocks, nsplit), dim3(256), 0, st, sa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.n1 = n1;
  int grid = n1;
  for (int i = 0; i < n; ++i) {
    a.lin[i].first2 = grid;
    grid += a.lin[i].n2;
  }
  if (grid == 0) return hipSuccess;
  // The persistent form wherever it fits.  Measured against the tiled form
  // with weights loaded non-temporally: faster on every 7B decode class at 1,
  // 8 and 64 tokens, o and gate,up at 32 (q,k,v at 32 within 3 %), and on
  // stage-2-only launches (13B tensor-parallel share at 64 tokens: each 2 us
  // faster; it loads its slice of t once, all at once, where a tiled-form
  // tile loads it a round at a time).
  PersArgs pa;
  int per = 0;
  if (plan_persistent(a, TB, &pa, &per)) {
    switch (TB) {
      case 1: return launch_pers<1>(pa, per, st);
      case 2: return launch_pers<2>(pa, per, st);
      default: return launch_pers<4>(pa, per, st);
    }
  }
  // Tiled form: a launch with fewer than kThinTiles 32-row stage-2 tiles
  // (o alone at 4096 outputs: 128) would leave half the CUs without V_r to
  // stream, so up to 32 tokens it takes 16-row tiles instead.
  constexpr int kThinTiles = 192;
  const bool thin = TB <= 2 && grid - n1 < kThinTiles;
  if (thin) {
    grid = n1;
    for (int i = 0; i < n; ++i) {
      LinArgs& L = a.lin[i];
      if (L.n2) L.n2 = (L.d_out + 15) / 16;
      L.first2 = grid;
      grid += L.n2;
    }
  }
  switch (TB) {
    case 1: return launch_decode<1>(a, grid, thin, st);
    case 2: return launch_decode<2>(a, grid, thin, st);
    default: return launch_decode<4>(a, grid, false, st);
  }
}

hipError_t decode_linear_bf16(const DecodeLinear& d, hipStream_t st) {
  return decode_group_bf16(&d, 1, st);
}

}  // namespace lr
