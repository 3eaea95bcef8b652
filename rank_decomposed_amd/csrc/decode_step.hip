// One decode step of a decoder layer whose linears are all decomposed, with a
// paged cache of rank-r latents that is reconstructed every step.
//
// DeInfer/en §1 (third bottleneck) and §2.C: decomposed models rebuild the KV
// cache while decoding by multiplying the cached low-rank rows by the upward
// projections; to keep that inside a static graph, a preparation stage on the
// host builds a remapping index list, and the replayed graph copies the rows
// into a compact buffer at a fixed address and runs one large fixed-size GEMM.
// The layer around it is LLaMA-shaped (MHA/GQA, GLU MLP; DeInfer/en §2.D).
//
// Every grid here is sized from fixed capacities (B, cap, max_seq_rows), never
// from live lengths: live counts (n_valid, seq_off, pos, slot_mapping, remap)
// are read from device buffers, so one captured graph serves every step.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "lowrank.h"
#include "lr_common.h"
#include "lr_kernels.h"

namespace lr {

namespace {

constexpr int kAttnChunk = 256;  // cached rows per attention workgroup

int64_t rup(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// ---------------------------------------------------------------- rotary table
// table[p][i] = (cos(p * theta^(-2i/hd)), sin(...)), computed in double.
__global__ void rope_table_kernel(float* table, int64_t max_pos, int half, double theta) {
  const int64_t n = max_pos * half;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t p = e / half;
    const int i = (int)(e % half);
    const double inv = pow(theta, -2.0 * i / (2.0 * half));
    double s, c;
    sincos((double)p * inv, &s, &c);
    table[2 * e] = (float)c;
    table[2 * e + 1] = (float)s;
  }
}

// ---------------------------------------------------------------- RMSNorm
// x[b] = bf16(h[b] / sqrt(mean(h[b]^2) + eps) * g), one workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int64_t ldh,
                                                      const uint16_t* __restrict__ g,
                                                      uint16_t* __restrict__ x, int64_t ldx, int d,
                                                      float eps) {
  __shared__ float red[256];
  const float* row = h + (int64_t)blockIdx.x * ldh;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss = fmaf(row[i], row[i], ss);
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const float scale = 1.0f / sqrtf(red[0] / (float)d + eps);
  uint16_t* out = x + (int64_t)blockIdx.x * ldx;
  for (int i = threadIdx.x; i < d; i += 256)
    out[i] = (uint16_t)f2bf(row[i] * scale * bf2f(g[i]));
}

// ---------------------------------------------------------------- append
// pool[slot[b], 0:r] = bf16(lat[b, 0:r]); out-of-range slots are skipped.
__global__ __launch_bounds__(256) void append_kernel(const float* __restrict__ lat, int64_t ldl,
                                                     int r, const int32_t* __restrict__ slot,
                                                     int64_t pool_rows, uint16_t* pool,
                                                     int64_t pool_ld) {
  const int b = blockIdx.x;
  const int64_t s = slot[b];
  if (s < 0 || s >= pool_rows) return;
  for (int j = threadIdx.x; j < r; j += 256)
    pool[s * pool_ld + j] = (uint16_t)f2bf(lat[(int64_t)b * ldl + j]);
}

// ---------------------------------------------------------------- SiLU * up
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ gate,
                                                       const uint16_t* __restrict__ up,
                                                       uint16_t* __restrict__ m, int64_t n) {
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const float gv = bf2f(gate[e]);
    const float s = gv / (1.0f + expf(-gv));
    m[e] = (uint16_t)f2bf(s * bf2f(up[e]));
  }
}

// ---------------------------------------------------------------- reconstruction
// rec[j, :] = buf[j, 0:r] . Vt^T for rows j < *n_valid: the fixed-size GEMM of
// the replay stage (DeInfer/en §2.C).  The grid covers the buffer capacity;
// tiles past n_valid exit.  With a rotary table, each head's pairs
// (c, c + hd/2) of row j are rotated by the row's position j - seq_off[i].
//
// A workgroup stages 128 rows of buf (all r columns, zero past r) in LDS once
// and sweeps every output column with 8 waves; wave (mh, nq) computes rows
// mh*64 .. +64 and 128 columns per 512-column chunk on MFMA 16x16x32, weight
// fragments streamed two k-steps ahead in registers.  The MFMA operands are
// swapped (weights as A) so each lane ends with 4 consecutive output columns
// of one row: rotary partners sit in the same lane and stores are 8 bytes.
constexpr int rBM = 128;          // latent rows per workgroup
constexpr int rNBW = 8;           // 16-column blocks per wave (128 columns)
constexpr int rMBW = 4;           // 16-row blocks per wave (64 rows)
constexpr int rChunk = 4 * rNBW * 16;  // 512 columns per sweep step
constexpr int rRing = 1;

struct ReconArgs {
  const uint16_t* a;  // [cap, lda] compact latents
  int64_t lda;
  const uint16_t* b;  // Vt [N, ldb]
  int64_t ldb;
  uint16_t* c;        // [cap, ldc]
  int64_t ldc;
  int cap, N, K, k_pad;
  const int32_t* n_valid;
  const float* rope;  // [max_pos, hd/2, 2] or null
  int64_t max_pos;
  int hd;
  const int32_t* seq_off;
  int B;
};

// LDS: latent tile [128][k_pad + 8] bf16, then (rotary only) the tile rows'
// cos/sin pairs as fp16x2 [128][hd/2] (|cos|, |sin| <= 1: fp16's 11-bit
// precision is below the bf16 rounding of the output)
size_t recon_lds_bytes(int64_t r, int64_t hd) {
  return (size_t)rBM * (rup(r, 32) + 8) * 2 + (size_t)rBM * (hd / 2) * 4;
}

// HD: head dimension when rotary is applied (64 or 128), 0 for none; a
// compile-time constant so the rotary pairing indexes registers statically.
template <int HD>
__global__ __launch_bounds__(512, 1) void recon_kernel(ReconArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int apitch = p.k_pad + 8;
  constexpr int half = HD / 2;
  uint16_t* as = smem;                                                  // [128][apitch]
  uint32_t* rcs = reinterpret_cast<uint32_t*>(smem + rBM * apitch);    // [128][half] fp16 cos|sin
  int nv = *p.n_valid;
  nv = nv < 0 ? 0 : (nv > p.cap ? p.cap : nv);
  const int m0 = blockIdx.x * rBM;
  if (m0 >= nv) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mh = wave >> 2, nq = wave & 3;
  const int rr = lane & 15, kq = (lane >> 4) * 8;

  // stage the latent tile, zero past K
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, view_bytes(p.cap, p.K, p.lda));
  const int kch = p.k_pad / 8;
  for (int e = threadIdx.x; e < rBM * kch; e += 512) {
    const int row = e / kch, k = (e % kch) * 8;
    u32x4 v = bload(ra, (uint32_t)(((int64_t)(m0 + row) * p.lda + k) * 2));
    if (k + 8 > p.K) v = mask_tail(v, k, p.K);
    *reinterpret_cast<u32x4*>(as + row * apitch + k) = v;
  }
  if (HD > 0) {
    for (int e = threadIdx.x; e < rBM * half; e += 512) {
      const int row = e / half, fi = e % half;
      const int j = m0 + row;
      int lo = 0, hi = p.B;  // i with seq_off[i] <= j < seq_off[i + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.seq_off[mid] <= j) lo = mid; else hi = mid;
      }
      int pos = j - p.seq_off[lo];
      pos = pos < 0 ? 0 : (pos >= p.max_pos ? (int)p.max_pos - 1 : pos);
      const float cs = p.rope[((int64_t)pos * half + fi) * 2];
      const float sn = p.rope[((int64_t)pos * half + fi) * 2 + 1];
      const _Float16 hc = (_Float16)cs, hs = (_Float16)sn;
      rcs[row * half + fi] = (uint32_t)__builtin_bit_cast(uint16_t, hc) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, hs) << 16);
    }
  }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b, view_bytes(p.N, p.K, p.ldb));
  const int ks = p.k_pad / 32;
  const bool tail = (p.K % 32) != 0;
  const int kf = tail ? ks - 1 : ks;
  for (int c0 = 0; c0 < p.N; c0 += rChunk) {
    const int n0 = c0 + nq * rNBW * 16;
    if (n0 >= p.N) continue;
    f32x4 acc[rNBW][rMBW];  // [column block][row block], C^T fragments
#pragma unroll
    for (int j = 0; j < rNBW; ++j)
#pragma unroll
      for (int i = 0; i < rMBW; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 bq[rRing][rNBW];
#pragma unroll
    for (int q = 0; q < rRing; ++q) frag_load<rNBW>(bq[q], rb, p.ldb, n0, q * 32, lane);
    int s = 0;
    for (; s + rRing <= kf; s += rRing) {
#pragma unroll
      for (int q = 0; q < rRing; ++q) {
        u32x4 a[rMBW];
#pragma unroll
        for (int i = 0; i < rMBW; ++i)
          a[i] = lds16(as + (mh * 64 + i * 16 + rr) * apitch + (s + q) * 32 + kq);
        frag_mma<rNBW, rMBW>(acc, bq[q], a);
        frag_load<rNBW>(bq[q], rb, p.ldb, n0, (s + q + rRing) * 32, lane);
      }
    }
#pragma unroll
    for (int q = 0; q < rRing; ++q) {
      if (s + q < kf || (tail && s + q == kf)) {
        if (s + q == kf) frag_mask<rNBW>(bq[q], kf * 32, p.K, lane);
        u32x4 a[rMBW];
#pragma unroll
        for (int i = 0; i < rMBW; ++i)
          a[i] = lds16(as + (mh * 64 + i * 16 + rr) * apitch + (s + q) * 32 + kq);
        frag_mma<rNBW, rMBW>(acc, bq[q], a);
      }
    }
    // lane holds rows (i*16 + rr) and columns n0 + j*16 + 4*(lane>>4) + v
#pragma unroll
    for (int i = 0; i < rMBW; ++i) {
      const int lrow = mh * 64 + i * 16 + rr;
      const int grow = m0 + lrow;
      if (HD > 0) {
        const uint32_t* tr = rcs + lrow * half;
        constexpr int hb = half / 16;  // column blocks per half head
#pragma unroll
        for (int j = 0; j < rNBW; ++j) {
          const int hc = (j * 16) % (HD > 0 ? HD : 1);  // block start inside its head
          if (hc >= half || j + hb >= rNBW) continue;  // rotated with its partner
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t w = tr[hc + 4 * (lane >> 4) + v];   // frequency index
            const float cs = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
            const float sn = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
            const float a0 = acc[j][i][v], b0 = acc[j + hb][i][v];
            acc[j][i][v] = a0 * cs - b0 * sn;
            acc[j + hb][i][v] = b0 * cs + a0 * sn;
          }
        }
      }
      if (grow < nv) {
#pragma unroll
        for (int j = 0; j < rNBW; ++j) {
          const int col = n0 + j * 16 + 4 * (lane >> 4);
          if (col < p.N) {
            const u32x2 w{pack_bf2(acc[j][i][0], acc[j][i][1]), pack_bf2(acc[j][i][2], acc[j][i][3])};
            *reinterpret_cast<u32x2*>(p.c + (int64_t)grow * p.ldc + col) = w;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- attention
// Partial softmax attention of one query (sequence i, head h) over one chunk
// of its packed rows [seq_off[i] + c*256, ...).  Output per chunk: running max
// m, sum l and unnormalised o[hd] (fp32).  K rows are already rotated.
template <int HD>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int64_t ldkv, const int32_t* __restrict__ seq_off,
    const int32_t* __restrict__ pos, const float* __restrict__ rope, int64_t max_pos, int H,
    int Hkv, int nch, int cap, float* __restrict__ part) {
  constexpr int HALF = HD / 2;
  __shared__ float qs[HD];
  __shared__ float sc[kAttnChunk];
  __shared__ float red[256];
  __shared__ float opart[256 / HALF][HD];
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const int beg = seq_off[i];
  int n = seq_off[i + 1] - beg;
  if (beg < 0 || beg >= cap) return;      // offsets are device data: stay inside cap
  n = n < cap - beg ? n : cap - beg;
  const int r0 = c * kAttnChunk;
  if (r0 >= n) return;
  const int cnt = min(kAttnChunk, n - r0);
  const int kvh = h / (H / Hkv);
  // rotated, scaled query
  if (threadIdx.x < HALF) {
    int p = pos[i];
    p = p < 0 ? 0 : (p >= max_pos ? (int)max_pos - 1 : p);
    const float cs = rope[((int64_t)p * HALF + threadIdx.x) * 2];
    const float sn = rope[((int64_t)p * HALF + threadIdx.x) * 2 + 1];
    const float a = bf2f(q[(int64_t)i * ldq + h * HD + threadIdx.x]);
    const float b = bf2f(q[(int64_t)i * ldq + h * HD + threadIdx.x + HALF]);
    const float scale = 1.0f / sqrtf((float)HD);
    qs[threadIdx.x] = (a * cs - b * sn) * scale;
    qs[threadIdx.x + HALF] = (b * cs + a * sn) * scale;
  }
  __syncthreads();
  // scores: thread t <-> row r0 + t
  float s = -INFINITY;
  if ((int)threadIdx.x < cnt) {
    const uint16_t* kr = K + (int64_t)(beg + r0 + threadIdx.x) * ldkv + kvh * HD;
    float acc = 0.f;
#pragma unroll
    for (int d0 = 0; d0 < HD; d0 += 8) {
      const u32x4 w = ldg16(kr + d0);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf2f(ww[e] & 0xffffu), qs[d0 + 2 * e], acc);
        acc = fmaf(bf2f(ww[e] >> 16), qs[d0 + 2 * e + 1], acc);
      }
    }
    s = acc;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + k]);
    __syncthreads();
  }
  const float m = red[0];
  __syncthreads();
  const float pexp = ((int)threadIdx.x < cnt) ? expf(s - m) : 0.f;
  sc[threadIdx.x] = pexp;
  red[threadIdx.x] = pexp;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  const float l = red[0];
  // o = sum_r p_r V_r: thread (pair dp, group g) walks rows g, g + G, ...
  constexpr int G = 256 / HALF;
  const int dp = threadIdx.x % HALF, g = threadIdx.x / HALF;
  float o0 = 0.f, o1 = 0.f;
  const uint16_t* vb = V + (int64_t)(beg + r0) * ldkv + kvh * HD + 2 * dp;
  for (int r = g; r < cnt; r += G) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(vb + (int64_t)r * ldkv);
    const float pr = sc[r];
    o0 = fmaf(pr, bf2f(w & 0xffffu), o0);
    o1 = fmaf(pr, bf2f(w >> 16), o1);
  }
  opart[g][2 * dp] = o0;
  opart[g][2 * dp + 1] = o1;
  __syncthreads();
  float* out = part + (((int64_t)i * H + h) * nch + c) * (HD + 2);
  if (threadIdx.x < HD) {
    float acc = 0.f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) acc += opart[gg][threadIdx.x];
    out[2 + threadIdx.x] = acc;
  }
  if (threadIdx.x == 0) {
    out[0] = m;
    out[1] = l;
  }
}

// Combine the chunks of (sequence i, head h): o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.
template <int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(const float* __restrict__ part, int H,
                                                          int nch,
                                                          const int32_t* __restrict__ seq_off,
                                                          int cap, uint16_t* __restrict__ o,
                                                          int64_t ldo) {
  const int h = blockIdx.x, i = blockIdx.y;
  const int beg = seq_off[i];
  int n = seq_off[i + 1] - beg;
  if (beg < 0 || beg >= cap) n = 0;
  n = n < cap - beg ? n : cap - beg;
  int used = (n + kAttnChunk - 1) / kAttnChunk;
  used = used < 0 ? 0 : (used > nch ? nch : used);
  const float* base = part + ((int64_t)i * H + h) * nch * (HD + 2);
  float M = -INFINITY;
  for (int c = 0; c < used; ++c) M = fmaxf(M, base[(int64_t)c * (HD + 2)]);
  float L = 0.f, acc = 0.f;
  for (int c = 0; c < used; ++c) {
    const float* pc = base + (int64_t)c * (HD + 2);
    const float w = expf(pc[0] - M);
    L = fmaf(w, pc[1], L);
    acc = fmaf(w, pc[2 + threadIdx.x], acc);
  }
  o[(int64_t)i * ldo + h * HD + threadIdx.x] = (uint16_t)f2bf(used > 0 ? acc / L : 0.f);
}

// ---------------------------------------------------------------- workspace
struct StepLayout {
  size_t lin, x, q, latk, latv, kbuf, vbuf, krec, vrec, part, o, gate, up, m, total;
  int64_t rk_ld, rv_ld, dkv, nch;
};

StepLayout step_layout(const lr_layer_weights* w, const lr_decode_state* s) {
  StepLayout L{};
  const int64_t B = s->B, d = w->d_model, dq = w->n_heads * w->head_dim;
  L.dkv = w->n_kv_heads * w->head_dim;
  L.rk_ld = rup(w->r[1], 8);
  L.rv_ld = rup(w->r[2], 8);
  L.nch = (s->max_seq_rows + kAttnChunk - 1) / kAttnChunk;
  const int64_t din[7] = {d, d, d, dq, d, d, w->d_ffn};
  const int64_t dout[7] = {dq, L.dkv, L.dkv, d, w->d_ffn, w->d_ffn, d};
  // the projections' scratch: q,k,v and gate,up go out as groups
  DecodeLinear g[7];
  for (int k = 0; k < 7; ++k) g[k] = DecodeLinear{B, din[k], w->r[k], dout[k]};
  size_t lin = decode_group_workspace_bytes(g, 3);
  lin = std::max(lin, decode_group_workspace_bytes(g + 4, 2));
  lin = std::max(lin, decode_workspace_bytes(B, din[3], w->r[3], dout[3]));
  lin = std::max(lin, decode_workspace_bytes(B, din[6], w->r[6], dout[6]));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = rup(off + bytes, 256);
    return at;
  };
  L.lin = take(lin);  // first: zero-filled once by the caller, kept zero by the kernels
  L.x = take(B * d * 2);
  L.q = take(B * dq * 2);
  L.latk = take(B * w->r[1] * 4);
  L.latv = take(B * w->r[2] * 4);
  L.kbuf = take(s->cap * L.rk_ld * 2);
  L.vbuf = take(s->cap * L.rv_ld * 2);
  L.krec = take(s->cap * L.dkv * 2);
  L.vrec = take(s->cap * L.dkv * 2);
  L.part = take(B * w->n_heads * L.nch * (w->head_dim + 2) * 4);
  L.o = take(B * dq * 2);
  L.gate = take(B * w->d_ffn * 2);
  L.up = take(B * w->d_ffn * 2);
  L.m = take(B * w->d_ffn * 2);
  L.total = off;
  return L;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

lr_status check_step(const lr_layer_weights* w, const lr_decode_state* s, const float* h) {
  if (!w || !s || !h) return LR_ERR_ARG;
  if (w->d_model <= 0 || w->n_heads <= 0 || w->n_kv_heads <= 0 || w->d_ffn <= 0) return LR_ERR_ARG;
  if (w->head_dim != 64 && w->head_dim != 128) return LR_ERR_UNSUPPORTED;
  if (w->n_heads % w->n_kv_heads) return LR_ERR_ARG;
  if (s->B <= 0 || s->cap <= 0 || s->max_seq_rows <= 0 || s->pool_rows <= 0) return LR_ERR_ARG;
  if (s->cap > INT32_MAX) return LR_ERR_ARG;
  if (s->B > 64) return LR_ERR_UNSUPPORTED;  // projections run on the decode path
  if (!w->rope || w->rope_max_pos <= 0 || !w->attn_norm || !w->ffn_norm) return LR_ERR_ARG;
  if (!s->k_pool || !s->v_pool || !s->slot_mapping || !s->remap || !s->seq_off || !s->pos ||
      !s->n_valid)
    return LR_ERR_ARG;
  const int64_t dq = w->n_heads * w->head_dim, dkv = w->n_kv_heads * w->head_dim;
  const int64_t din[7] = {w->d_model, w->d_model, w->d_model, dq, w->d_model, w->d_model, w->d_ffn};
  const int64_t dout[7] = {dq, dkv, dkv, w->d_model, w->d_ffn, w->d_ffn, w->d_model};
  for (int k = 0; k < 7; ++k) {
    if (!w->Ut[k] || !w->Vt[k] || w->r[k] <= 0) return LR_ERR_ARG;
    if (w->ldu[k] < din[k] || w->ldv[k] < w->r[k]) return LR_ERR_ARG;
    if (!al16(w->Ut[k]) || !al16(w->Vt[k]) || w->ldu[k] % 8 || w->ldv[k] % 8) return LR_ERR_ALIGN;
    if (w->ldu[k] >= (1 << 24) || w->ldv[k] >= (1 << 24) || din[k] >= (1 << 24))
      return LR_ERR_UNSUPPORTED;
  }
  if (s->pool_ld < w->r[1] || s->pool_ld < w->r[2]) return LR_ERR_ARG;
  // the reconstruction keeps a 128-row latent tile in LDS
  if (recon_lds_bytes(w->r[1], w->head_dim) > 163840 ||
      recon_lds_bytes(w->r[2], w->head_dim) > 163840)
    return LR_ERR_UNSUPPORTED;
  if (!al16(s->k_pool) || !al16(s->v_pool) || s->pool_ld % 8) return LR_ERR_ALIGN;
  if (w->d_model % 8 || w->d_ffn % 8) return LR_ERR_ALIGN;
  return LR_OK;
}

}  // namespace

}  // namespace lr

using namespace lr;

extern "C" lr_status lowrank_rope_table(int64_t head_dim, int64_t max_pos, float theta,
                                        float* table, hipStream_t stream) {
  if (head_dim <= 0 || head_dim % 2 || max_pos <= 0 || !table || !(theta > 0.f)) return LR_ERR_ARG;
  const int64_t n = max_pos * (head_dim / 2);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, stream, table, max_pos,
                     (int)(head_dim / 2), (double)theta);
  return hipGetLastError() == hipSuccess ? LR_OK : LR_ERR_HIP;
}

extern "C" size_t lowrank_decode_step_workspace_bytes(const lr_layer_weights* w,
                                                      const lr_decode_state* s) {
  if (!w || !s || s->B <= 0 || s->cap <= 0 || s->max_seq_rows <= 0) return 0;
  return step_layout(w, s).total;
}

extern "C" lr_status lowrank_layer_decode_step(const lr_layer_weights* w,
                                               const lr_decode_state* s, float* h,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t st) {
  const lr_status chk = check_step(w, s, h);
  if (chk != LR_OK) return chk;
  const StepLayout L = step_layout(w, s);
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return LR_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const int B = (int)s->B;
  const int64_t d = w->d_model, dq = w->n_heads * w->head_dim, ffn = w->d_ffn;
  uint16_t* x = reinterpret_cast<uint16_t*>(ws + L.x);
  uint16_t* q = reinterpret_cast<uint16_t*>(ws + L.q);
  float* latk = reinterpret_cast<float*>(ws + L.latk);
  float* latv = reinterpret_cast<float*>(ws + L.latv);
  uint16_t* kbuf = reinterpret_cast<uint16_t*>(ws + L.kbuf);
  uint16_t* vbuf = reinterpret_cast<uint16_t*>(ws + L.vbuf);
  uint16_t* krec = reinterpret_cast<uint16_t*>(ws + L.krec);
  uint16_t* vrec = reinterpret_cast<uint16_t*>(ws + L.vrec);
  float* part = reinterpret_cast<float*>(ws + L.part);
  uint16_t* o = reinterpret_cast<uint16_t*>(ws + L.o);
  uint16_t* gate = reinterpret_cast<uint16_t*>(ws + L.gate);
  uint16_t* up = reinterpret_cast<uint16_t*>(ws + L.up);
  uint16_t* m = reinterpret_cast<uint16_t*>(ws + L.m);
  void* lin = ws + L.lin;
  hipError_t e = hipSuccess;
#define LR_CHECK(expr)                \
  do {                                \
    e = (expr);                       \
    if (e != hipSuccess) return LR_ERR_HIP; \
  } while (0)

  auto linear = [&](int k, const void* in, int64_t din, int64_t ldin, int64_t dout, void* y,
                    float* yacc, float* t_out) -> DecodeLinear {
    DecodeLinear dl{};
    dl.T = B;
    dl.d_in = din;
    dl.r = w->r[k];
    dl.d_out = dout;
    dl.x = in;
    dl.ldx = ldin;
    dl.Ut = w->Ut[k];
    dl.ldu = w->ldu[k];
    dl.Vt = w->Vt[k];
    dl.ldv = w->ldv[k];
    dl.y = y;
    dl.ldy = dout;
    dl.t_io = t_out;
    dl.ldt = w->r[k];
    dl.flags = t_out ? 1u : 0u;
    dl.workspace = lin;
    dl.y_acc = yacc;
    dl.ld_acc = d;
    return dl;
  };

  // attention block
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(B), dim3(256), 0, st, h, d,
                     static_cast<const uint16_t*>(w->attn_norm), x, d, (int)d, w->eps);
  LR_CHECK(hipGetLastError());
  {
    // q (full) and the k, v latents (stage 1 only) read the same x: one launch
    const DecodeLinear qkv[3] = {linear(0, x, d, d, dq, q, nullptr, nullptr),
                                 linear(1, x, d, d, L.dkv, nullptr, nullptr, latk),
                                 linear(2, x, d, d, L.dkv, nullptr, nullptr, latv)};
    LR_CHECK(decode_group_bf16(qkv, 3, st));
  }
  hipLaunchKernelGGL(append_kernel, dim3(B), dim3(256), 0, st, latk, w->r[1], (int)w->r[1],
                     s->slot_mapping, s->pool_rows, static_cast<uint16_t*>(s->k_pool), s->pool_ld);
  LR_CHECK(hipGetLastError());
  hipLaunchKernelGGL(append_kernel, dim3(B), dim3(256), 0, st, latv, w->r[2], (int)w->r[2],
                     s->slot_mapping, s->pool_rows, static_cast<uint16_t*>(s->v_pool), s->pool_ld);
  LR_CHECK(hipGetLastError());
  LR_CHECK(remap_gather(2, s->k_pool, s->pool_rows, s->pool_ld, s->remap, s->cap, s->n_valid,
                        w->r[1], kbuf, L.rk_ld, st));
  LR_CHECK(remap_gather(2, s->v_pool, s->pool_rows, s->pool_ld, s->remap, s->cap, s->n_valid,
                        w->r[2], vbuf, L.rv_ld, st));
  ReconArgs ra{};
  ra.cap = (int)s->cap;
  ra.N = (int)L.dkv;
  ra.n_valid = s->n_valid;
  ra.max_pos = w->rope_max_pos;
  ra.hd = (int)w->head_dim;
  ra.seq_off = s->seq_off;
  ra.B = B;
  const dim3 rgrid((unsigned)((s->cap + rBM - 1) / rBM));
  for (int kv = 0; kv < 2; ++kv) {
    const int64_t r = w->r[1 + kv];
    ra.a = kv ? vbuf : kbuf;
    ra.lda = kv ? L.rv_ld : L.rk_ld;
    ra.b = static_cast<const uint16_t*>(w->Vt[1 + kv]);
    ra.ldb = w->ldv[1 + kv];
    ra.c = kv ? vrec : krec;
    ra.ldc = L.dkv;
    ra.K = (int)r;
    ra.k_pad = (int)rup(r, 32);
    ra.rope = kv ? nullptr : w->rope;
    const size_t lds = recon_lds_bytes(r, kv ? 0 : w->head_dim);
    static std::once_flag lds_once;  // raise the dynamic-LDS limit once per process
    std::call_once(lds_once, [] {
      (void)hipFuncSetAttribute((const void*)recon_kernel<0>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
      (void)hipFuncSetAttribute((const void*)recon_kernel<64>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
      (void)hipFuncSetAttribute((const void*)recon_kernel<128>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
    });
    if (kv)
      hipLaunchKernelGGL(recon_kernel<0>, rgrid, dim3(512), lds, st, ra);
    else if (w->head_dim == 128)
      hipLaunchKernelGGL(recon_kernel<128>, rgrid, dim3(512), lds, st, ra);
    else
      hipLaunchKernelGGL(recon_kernel<64>, rgrid, dim3(512), lds, st, ra);
    LR_CHECK(hipGetLastError());
  }
  const dim3 agrid((unsigned)L.nch, (unsigned)w->n_heads, (unsigned)B);
  if (w->head_dim == 128) {
    hipLaunchKernelGGL(attn_partial_kernel<128>, agrid, dim3(256), 0, st, q, dq, krec, vrec,
                       L.dkv, s->seq_off, s->pos, w->rope, w->rope_max_pos, (int)w->n_heads,
                       (int)w->n_kv_heads, (int)L.nch, (int)s->cap, part);
    LR_CHECK(hipGetLastError());
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((unsigned)w->n_heads, (unsigned)B),
                       dim3(128), 0, st, part, (int)w->n_heads, (int)L.nch, s->seq_off, (int)s->cap, o, dq);
  } else {
    hipLaunchKernelGGL(attn_partial_kernel<64>, agrid, dim3(256), 0, st, q, dq, krec, vrec,
                       L.dkv, s->seq_off, s->pos, w->rope, w->rope_max_pos, (int)w->n_heads,
                       (int)w->n_kv_heads, (int)L.nch, (int)s->cap, part);
    LR_CHECK(hipGetLastError());
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)w->n_heads, (unsigned)B),
                       dim3(64), 0, st, part, (int)w->n_heads, (int)L.nch, s->seq_off, (int)s->cap, o, dq);
  }
  LR_CHECK(hipGetLastError());
  LR_CHECK(decode_linear_bf16(linear(3, o, dq, dq, d, nullptr, h, nullptr), st));
  // MLP block
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(B), dim3(256), 0, st, h, d,
                     static_cast<const uint16_t*>(w->ffn_norm), x, d, (int)d, w->eps);
  LR_CHECK(hipGetLastError());
  {
    const DecodeLinear gu[2] = {linear(4, x, d, d, ffn, gate, nullptr, nullptr),
                                linear(5, x, d, d, ffn, up, nullptr, nullptr)};
    LR_CHECK(decode_group_bf16(gu, 2, st));
  }
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((B * ffn + 255) / 256 < 4096 ? (B * ffn + 255) / 256 : 4096)),
                     dim3(256), 0, st, gate, up, m, (int64_t)B * ffn);
  LR_CHECK(hipGetLastError());
  LR_CHECK(decode_linear_bf16(linear(6, m, ffn, ffn, d, nullptr, h, nullptr), st));
#undef LR_CHECK
  return LR_OK;
}
