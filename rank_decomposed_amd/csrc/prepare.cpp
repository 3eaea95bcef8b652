// Host-side preparation stage of the paged latent cache (DeInfer/en §2.C
// "Preparation Stage"; DeInfer/zh remapping table; DeInfer/es §2 "Etapa de
// Preparación"): walk each sequence's block table, merge physically
// consecutive blocks into runs, and emit the remapping index list that the
// in-graph gather follows, plus the per-sequence offsets, positions and the
// slots of the tokens being decoded.  Runs on the CPU between graph replays;
// the caller copies the arrays into fixed device buffers.
#include <stdint.h>

#include "lowrank.h"

extern "C" lr_status lowrank_prepare_decode(int64_t B, const int32_t* lengths,
                                            const int32_t* tables, int64_t table_ld,
                                            int64_t block, int64_t cap, int32_t* remap,
                                            int32_t* seq_off, int32_t* pos,
                                            int32_t* slot_mapping, int32_t* n_valid,
                                            int32_t* n_runs, int32_t* runs, int64_t max_runs) {
  if (B < 0 || block <= 0 || cap < 0 || table_ld < 0) return LR_ERR_ARG;
  if (!remap || !seq_off || !n_valid || !n_runs) return LR_ERR_ARG;
  if (B > 0 && (!lengths || !tables || !pos || !slot_mapping)) return LR_ERR_ARG;
  if (runs && max_runs < 0) return LR_ERR_ARG;

  // offsets first: reject before writing anything else
  int64_t off = 0;
  for (int64_t i = 0; i < B; ++i) {
    const int64_t L = lengths[i];
    if (L < 0) return LR_ERR_ARG;
    const int64_t nblk = (L + 1 + block - 1) / block;
    if (nblk > table_ld) return LR_ERR_ARG;
    off += L + 1;
    if (off > INT32_MAX) return LR_ERR_CAPACITY;
  }
  if (off > cap) return LR_ERR_CAPACITY;
  for (int64_t i = 0; i < B; ++i) {
    const int32_t* t = tables + i * table_ld;
    const int64_t nblk = (lengths[i] + 1 + block - 1) / block;
    for (int64_t b = 0; b < nblk; ++b)
      if (t[b] < 0 || (int64_t)t[b] * block + block - 1 > INT32_MAX) return LR_ERR_ARG;
  }

  int64_t nr = 0;
  off = 0;
  seq_off[0] = 0;
  for (int64_t i = 0; i < B; ++i) {
    const int32_t* t = tables + i * table_ld;
    const int64_t n = (int64_t)lengths[i] + 1;
    const int64_t nblk = (n + block - 1) / block;
    int64_t b = 0;
    while (b < nblk) {
      int64_t e = b + 1;
      while (e < nblk && t[e] == t[e - 1] + 1) ++e;
      const int64_t lo = b * block;
      const int64_t hi = (e * block < n) ? e * block : n;
      const int64_t src = (int64_t)t[b] * block;
      if (runs) {
        if (nr >= max_runs) return LR_ERR_CAPACITY;
        runs[3 * nr + 0] = (int32_t)src;
        runs[3 * nr + 1] = (int32_t)(off + lo);
        runs[3 * nr + 2] = (int32_t)(hi - lo);
      }
      for (int64_t p = lo; p < hi; ++p) remap[off + p] = (int32_t)(src + (p - lo));
      ++nr;
      b = e;
    }
    const int64_t L = lengths[i];
    pos[i] = (int32_t)L;
    slot_mapping[i] = (int32_t)((int64_t)t[L / block] * block + L % block);
    off += n;
    seq_off[i + 1] = (int32_t)off;
  }
  for (int64_t j = off; j < cap; ++j) remap[j] = -1;
  *n_valid = (int32_t)off;
  *n_runs = (int32_t)nr;
  return LR_OK;
}
