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
// One kernel per projection; the grid holds every stage-1 tile and then every
// stage-2 tile, tile = blockIdx.x.  Workgroups are dispatched to each XCD in
// index order and stage-1 tiles never wait, so a waiting stage-2 tile can
// never hold resources that a stage-1 tile it waits for still needs.
//   stage-1 tile: RT weight rows of U_r^T x one K range.  The 4 waves split
//     the K range, are reduced through LDS, and with several K ranges per row
//     tile the partials meet in the workspace; the last to arrive sums them in
//     K-range order (deterministic) and publishes t (fp32 for t_io, bf16 for
//     stage 2; for T <= 16 also the bf16 residual t - bf16(t), so stage 2 sees
//     ~16 mantissa bits at the cost of a second MFMA).
//   stage-2 tile: RT rows of V_r^T x one K range.  It issues the loads of its
//     first round of V_r fragments *before* waiting for t, so the V_r stream
//     overlaps stage 1; then it waits for the "t ready" flag, reads t and
//     finishes like a stage-1 tile, writing y in bf16.
// Synchronisation avoids cache-wide operations and hot addresses:
//   * data that crosses workgroups (stage-1 partials, the published t) is
//     written with device-coherent stores and the writer waits for their
//     completion before it bumps a counter, so no L2 write-back is needed;
//     partials are read back with device-coherent loads, and a stage-2 tile
//     issues one device-scope acquire (L1/L2 invalidate) before reading t;
//   * device-scope atomics on one address serialise (~10 ns each on this
//     part), so producers count on one cache line, the last producer raises a
//     flag on another line, and waiting tiles poll only the flag.
// Counters live in the workspace and are returned to zero by the last
// workgroup, so consecutive calls (and graph replays) need no memset.  Every
// wait is bounded: past ~1 s it records an error flag and proceeds.
#include <algorithm>

#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int kWaves = 4;
constexpr uint32_t kSpinLimit = 1u << 22;

// control block (uint32 words) at the start of the workspace; each hot word
// on a cache line of its own
enum { CTL_DONE = 0, CTL_TREADY = 32, CTL_GO = 64, CTL_ERR = 96, CTL_CNT = 128 };

struct DecArgs {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* ut;
  int64_t ldu;
  const uint16_t* vt;
  int64_t ldv;
  uint16_t* y;
  int64_t ldy;
  float* yacc;  // optional: yacc[T, ldacc] += y (fp32) instead of writing y
  int64_t ldacc;
  float* t32;  // optional fp32 t [T, ldt32] (stage-1 output)
  int64_t ldt32;
  uint16_t* thi;  // bf16 t [T, ldtb]
  uint16_t* tlo;  // bf16 residual (T <= 16)
  int64_t ldtb;
  float* part;     // partial tiles of both stages
  uint32_t* ctl;   // control block + per-row-tile arrival counters
  int T, d_in, r, d_out;
  int nrt1, S1, kc1;  // stage 1: row tiles, K ranges, K range width
  int nrt2, S2, kc2;  // stage 2
  int64_t part2_off;  // float offset of stage-2 partials in part
  int t_ready_target; // stage-1 row tiles that publish t before stage 2 may start
};

// Relaxed device-scope atomics: on gfx950 these are plain loads/stores with
// device coherence (no cache maintenance); ordering is made explicit with a
// wait for outstanding memory operations before a counter is bumped.
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_relaxed(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until every memory operation this thread issued has completed
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void store_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One tile: rows [row0, row0 + 16*RB) of B, K range [kbeg, kend); each wave
// takes a contiguous run of 32-wide k-steps and walks it KSW steps at a time.
// Result (reduced over the 4 waves) left in LDS as red[NREG][64] with
// element (reg, lane) -> token tb*16 + 4*(lane>>4) + v, row row0 + rb*16 + (lane&15),
// reg = (tb*RB + rb)*4 + v.
template <int TB, int RB, int KSW, bool SPLIT, bool WAIT>
__device__ void tile_product(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Alo,
                             int64_t lda, const uint16_t* __restrict__ B, int64_t ldb, int T,
                             int N, int row0, int kbeg, int kend, float* red, uint32_t* ctl,
                             int ready_target) {
  // RB 16-row blocks per wave; all 4 waves share the rows and split K
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rr = lane & 15;
  const int kq = (lane >> 4) * 8;

  const int nsteps = (kend - kbeg + 31) / 32;
  const int per = (nsteps + kWaves - 1) / kWaves;  // contiguous k-steps per wave
  const int s_lo = wave * per;
  const int s_hi = min(nsteps, s_lo + per);

  const uint16_t* brow[RB];
  bool bok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + rb * 16 + rr;
    bok[rb] = row < N;
    brow[rb] = B + (int64_t)(bok[rb] ? row : 0) * ldb;
  }
  const uint16_t* arow[TB];
  const uint16_t* alrow[TB];
  bool aok[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int tok = tb * 16 + rr;
    aok[tb] = tok < T;
    arow[tb] = A + (int64_t)(aok[tb] ? tok : 0) * lda;
    alrow[tb] = SPLIT ? Alo + (int64_t)(aok[tb] ? tok : 0) * lda : nullptr;
  }

  f32x4 acc[TB][RB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[tb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool waited = !WAIT;
  for (int s0 = s_lo; s0 < s_hi || !waited; s0 += KSW) {
    u32x4 bv[KSW][RB];
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int s = s0 + i;
      const int k = kbeg + s * 32 + kq;
      const bool kin = s < s_hi && k < kend;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (kin && bok[rb]) {
          v = ldg16_stream(brow[rb] + k);
          if (k + 8 > kend) v = mask_tail(v, k, kend);
        }
        bv[i][rb] = v;
      }
    }
    if (!waited) {
      // the first round of weights is in flight; now wait for t
      if (threadIdx.x == 0 && ready_target > 0) {
        uint32_t spins = 0;
        while (load_relaxed(ctl + CTL_GO) == 0u) {
          __builtin_amdgcn_s_sleep(8);
          if (++spins > kSpinLimit) {
            store_relaxed(ctl + CTL_ERR, 1u);
            break;
          }
        }
        fence_acquire();
      }
      __syncthreads();
      waited = true;
    }
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int s = s0 + i;
      // wave-uniform skip only: MFMA reads every lane's operands, so lanes
      // past kend take part with zero-filled fragments
      if (s >= s_hi) continue;
      const int k = kbeg + s * 32 + kq;
      const bool kin = k < kend;
      u32x4 av[TB], alv[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        av[tb] = (kin && aok[tb]) ? ldg16(arow[tb] + k) : u32x4{0, 0, 0, 0};
        if (SPLIT) alv[tb] = (kin && aok[tb]) ? ldg16(alrow[tb] + k) : u32x4{0, 0, 0, 0};
        if (kin && k + 8 > kend) {
          av[tb] = mask_tail(av[tb], k, kend);
          if (SPLIT) alv[tb] = mask_tail(alv[tb], k, kend);
        }
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[tb][rb] = mfma16x16x32(av[tb], bv[i][rb], acc[tb][rb]);
          if (SPLIT) acc[tb][rb] = mfma16x16x32(alv[tb], bv[i][rb], acc[tb][rb]);
        }
    }
    if (s0 >= s_hi) break;  // wait-only round of an idle wave
  }

  // reduce the 4 waves: ((w0 + w2) + (w1 + w3)), fixed order
  constexpr int NREG = TB * RB * 4;
  float* buf0 = red;               // [NREG][64]
  float* buf1 = red + NREG * 64;   // [NREG][64]
  if (wave >= 2) {
    float* b = wave == 2 ? buf0 : buf1;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) b[((tb * RB + rb) * 4 + v) * 64 + lane] = acc[tb][rb][v];
  }
  __syncthreads();
  if (wave < 2) {
    float* b = wave == 0 ? buf0 : buf1;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[tb][rb][v] += b[((tb * RB + rb) * 4 + v) * 64 + lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) buf1[((tb * RB + rb) * 4 + v) * 64 + lane] = acc[tb][rb][v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int e = ((tb * RB + rb) * 4 + v) * 64 + lane;
          buf0[e] = acc[tb][rb][v] + buf1[e];
        }
  }
  __syncthreads();
}

// Map a flat result element e = reg*64 + lane to (token, row offset).
template <int RB>
__device__ __forceinline__ void elem_coords(int e, int* tok, int* row) {
  const int reg = e >> 6, lane = e & 63;
  const int v = reg & 3, rb = (reg >> 2) % RB, tb = (reg >> 2) / RB;
  *tok = tb * 16 + 4 * (lane >> 4) + v;
  *row = rb * 16 + (lane & 15);
}

// Stage epilogue: sum split-K partials if needed, then write t (stage 1) or
// y (stage 2).  Called by every thread of the workgroup.
template <int TB, int RB, bool SPLIT, bool STAGE1>
__device__ void finish_tile(const DecArgs& p, float* red, int rt, int s, int S, int row0,
                            uint32_t* sh_flag) {
  constexpr int NREG = TB * RB * 4;
  float* part = STAGE1 ? p.part : p.part + p.part2_off;
  uint32_t* cnt = p.ctl + CTL_CNT + (STAGE1 ? 0 : p.nrt1);
  bool final_tile = true;
  if (S > 1) {
    float* mine = part + ((int64_t)rt * S + s) * (NREG * 64);
    for (int e = threadIdx.x; e < NREG * 64; e += 256) store_coherent(mine + e, red[e]);
    wait_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = atomic_add_agent(cnt + rt, 1u);
      *sh_flag = (old == (uint32_t)(S - 1)) ? 1u : 0u;
      if (*sh_flag) store_relaxed(cnt + rt, 0u);  // every sibling has arrived
    }
    __syncthreads();
    final_tile = *sh_flag != 0;
    if (final_tile) {
      const float* base = part + (int64_t)rt * S * (NREG * 64);
      for (int e = threadIdx.x; e < NREG * 64; e += 256) {
        float v = 0.f;
        for (int j = 0; j < S; ++j) v += load_coherent(base + (int64_t)j * (NREG * 64) + e);
        red[e] = v;
      }
      __syncthreads();
    }
  }
  if (!final_tile) return;
  const int N = STAGE1 ? p.r : p.d_out;
  for (int e = threadIdx.x; e < NREG * 64; e += 256) {
    int tok, ro;
    elem_coords<RB>(e, &tok, &ro);
    const int n = row0 + ro;
    if (tok >= p.T || n >= N) continue;
    const float v = red[e];
    if (STAGE1) {
      if (p.t32) p.t32[(int64_t)tok * p.ldt32 + n] = v;
      const uint32_t hi = f2bf(v);
      store_coherent(p.thi + (int64_t)tok * p.ldtb + n, (uint16_t)hi);
      if (SPLIT) store_coherent(p.tlo + (int64_t)tok * p.ldtb + n, (uint16_t)f2bf(v - bf2f(hi)));
    } else if (p.yacc) {
      p.yacc[(int64_t)tok * p.ldacc + n] += v;   // each element owned by one tile
    } else {
      p.y[(int64_t)tok * p.ldy + n] = (uint16_t)f2bf(v);
    }
  }
  if (STAGE1) {
    wait_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = atomic_add_agent(p.ctl + CTL_TREADY, 1u);
      if (old == (uint32_t)(p.t_ready_target - 1)) store_relaxed(p.ctl + CTL_GO, 1u);
    }
  }
}

template <int TB, int RB1, int RB2, int KSW, bool SPLIT>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs p) {
  constexpr int NREG = TB * (RB1 > RB2 ? RB1 : RB2) * 4;
  __shared__ float red[2 * NREG * 64];
  __shared__ uint32_t sh_flag;

  const int n1 = p.nrt1 * p.S1, n2 = p.nrt2 * p.S2;
  const int tile = (int)blockIdx.x;
  if (tile < n1) {
    const int rt = tile / p.S1, s = tile % p.S1;
    const int kbeg = s * p.kc1, kend = min(p.d_in, kbeg + p.kc1);
    tile_product<TB, RB1, KSW, false, false>(p.x, nullptr, p.ldx, p.ut, p.ldu, p.T, p.r,
                                             rt * 16 * RB1, kbeg, kend, red, p.ctl, 0);
    finish_tile<TB, RB1, SPLIT, true>(p, red, rt, s, p.S1, rt * 16 * RB1, &sh_flag);
  } else {
    const int t2 = tile - n1;
    const int rt = t2 / p.S2, s = t2 % p.S2;
    const int kbeg = s * p.kc2, kend = min(p.r, kbeg + p.kc2);
    tile_product<TB, RB2, KSW, SPLIT, true>(p.thi, p.tlo, p.ldtb, p.vt, p.ldv, p.T, p.d_out,
                                            rt * 16 * RB2, kbeg, kend, red, p.ctl,
                                            p.t_ready_target);
    finish_tile<TB, RB2, SPLIT, false>(p, red, rt, s, p.S2, rt * 16 * RB2, &sh_flag);
  }

  // the last workgroup to finish returns the counters to zero
  if (threadIdx.x == 0) {
    const uint32_t total = (uint32_t)(n1 + n2);
    const uint32_t old = atomic_add_agent(p.ctl + CTL_DONE, 1u);
    if (old == total - 1) {
      store_relaxed(p.ctl + CTL_TREADY, 0u);
      store_relaxed(p.ctl + CTL_GO, 0u);
      store_relaxed(p.ctl + CTL_DONE, 0u);
    }
  }
}

// t (fp32, caller's layout) -> bf16 (and bf16 residual) for a stage-2-only call.
__global__ __launch_bounds__(256) void split_t_kernel(const float* __restrict__ t, int64_t ldt,
                                                      int T, int N, uint16_t* thi, uint16_t* tlo,
                                                      int64_t ldtb) {
  const int64_t total = (int64_t)T * ldtb;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int tok = (int)(e / ldtb), n = (int)(e % ldtb);
    if (n >= N) continue;
    const float v = t[(int64_t)tok * ldt + n];
    const uint32_t hi = f2bf(v);
    thi[e] = (uint16_t)hi;
    if (tlo) tlo[e] = (uint16_t)f2bf(v - bf2f(hi));
  }
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Tiling of one call; identical on the sizing and launch sides.
struct Plan {
  int TB, RB1, RB2;
  int nrt1, S1, kc1, nrt2, S2, kc2;
  int64_t ldtb;
  size_t off_part, part2_off_floats, off_thi, off_tlo, bytes;
};

Plan make_plan(int64_t T, int64_t d_in, int64_t r, int64_t d_out) {
  Plan pl{};
  pl.TB = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  pl.RB1 = pl.TB;                   // activation re-reads ~ T / (16 RB1) of the weight bytes
  pl.RB2 = pl.TB == 4 ? 2 : pl.TB;
  // stage 1: split K until ~512 tiles are in flight, but keep each K range
  // >= kc_min so the fp32 partials stay a small fraction of the weight bytes
  const int RT1 = 16 * pl.RB1;
  pl.nrt1 = (int)((r + RT1 - 1) / RT1);
  const int kc_min = pl.TB == 1 ? 128 : 512;
  int S1 = (int)((512 + pl.nrt1 - 1) / pl.nrt1);
  int kc1 = (int)round_up((d_in + S1 - 1) / S1, 128);
  if (kc1 < kc_min) kc1 = kc_min;
  S1 = (int)((d_in + kc1 - 1) / kc1);
  pl.S1 = S1;
  pl.kc1 = kc1;
  // stage 2: one tile per row block, whole K (several register rounds)
  const int RT2 = 16 * pl.RB2;
  pl.nrt2 = (int)((d_out + RT2 - 1) / RT2);
  pl.S2 = 1;
  pl.kc2 = (int)round_up(r, 32);
  pl.ldtb = round_up(r, 8);
  const size_t tile1 = (size_t)pl.TB * pl.RB1 * 4 * 64, tile2 = (size_t)pl.TB * pl.RB2 * 4 * 64;
  const size_t p1 = pl.S1 > 1 ? (size_t)pl.nrt1 * pl.S1 * tile1 : 0;
  const size_t p2 = pl.S2 > 1 ? (size_t)pl.nrt2 * pl.S2 * tile2 : 0;
  const size_t ctl_bytes = round_up(4 * (CTL_CNT + pl.nrt1 + pl.nrt2), 256);
  pl.off_part = ctl_bytes;
  pl.part2_off_floats = p1;
  pl.off_thi = round_up(pl.off_part + (p1 + p2) * 4, 256);
  const size_t tb_bytes = round_up(T * pl.ldtb * 2, 256);
  pl.off_tlo = pl.off_thi + tb_bytes;
  pl.bytes = pl.off_tlo + tb_bytes;
  return pl;
}

template <int TB, int RB1, int RB2>
hipError_t launch_decode(const DecArgs& a, int grid, hipStream_t st) {
  constexpr int KSW = 8 / TB;
  hipLaunchKernelGGL((decode_kernel<TB, RB1, RB2, KSW, TB == 1>), dim3(grid), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int64_t T, int64_t d_in, int64_t r, int64_t d_out) {
  return make_plan(T, d_in, r, d_out).bytes;
}

hipError_t decode_linear_bf16(const DecodeLinear& d, hipStream_t st) {
  const Plan pl = make_plan(d.T, d.d_in, d.r, d.d_out);
  char* ws = static_cast<char*>(d.workspace);
  DecArgs a{};
  a.x = static_cast<const uint16_t*>(d.x);
  a.ldx = d.ldx;
  a.ut = static_cast<const uint16_t*>(d.Ut);
  a.ldu = d.ldu;
  a.vt = static_cast<const uint16_t*>(d.Vt);
  a.ldv = d.ldv;
  a.y = static_cast<uint16_t*>(d.y);
  a.ldy = d.ldy;
  a.yacc = d.y_acc;
  a.ldacc = d.ld_acc;
  a.t32 = d.t_io;
  a.ldt32 = d.ldt;
  a.thi = reinterpret_cast<uint16_t*>(ws + pl.off_thi);
  a.tlo = reinterpret_cast<uint16_t*>(ws + pl.off_tlo);
  a.ldtb = pl.ldtb;
  a.part = reinterpret_cast<float*>(ws + pl.off_part);
  a.ctl = reinterpret_cast<uint32_t*>(ws);
  a.T = (int)d.T;
  a.d_in = (int)d.d_in;
  a.r = (int)d.r;
  a.d_out = (int)d.d_out;
  a.nrt1 = pl.nrt1;
  a.S1 = pl.S1;
  a.kc1 = pl.kc1;
  a.nrt2 = pl.nrt2;
  a.S2 = pl.S2;
  a.kc2 = pl.kc2;
  a.part2_off = (int64_t)pl.part2_off_floats;
  a.t_ready_target = pl.nrt1;

  if (d.flags == 1) {  // stage 1 only
    a.nrt2 = 0;
  } else if (d.flags == 2) {  // stage 2 only: t from t_io
    const int64_t total = d.T * pl.ldtb;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(split_t_kernel, dim3(blocks), dim3(256), 0, st, d.t_io, d.ldt, (int)d.T,
                       (int)d.r, a.thi, pl.TB == 1 ? a.tlo : (uint16_t*)nullptr, pl.ldtb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.nrt1 = 0;
    a.t_ready_target = 0;
  }
  const int grid = a.nrt1 * a.S1 + a.nrt2 * a.S2;
  switch (pl.TB) {
    case 1: return launch_decode<1, 1, 1>(a, grid, st);
    case 2: return launch_decode<2, 2, 2>(a, grid, st);
    default: return launch_decode<4, 4, 2>(a, grid, st);
  }
}

}  // namespace lr
