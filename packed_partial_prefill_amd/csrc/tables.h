// Device side of the per-call tables of a layer repair (LayerTables): the
// attention plan of "Budgeted KV-Cache Repair", section 13.2, Eq. 23-24, and
// the RoPE table of each packed row's global position.
#pragma once

#include "common.h"
#include "kvr_internal.h"

namespace kvr {

// Attention plan entry t: first KV tile only partly visible to query tile t
// (n_full) and tiles it needs (n_total).
__device__ __forceinline__ void plan_entry(const int32_t* __restrict__ T, int B, int group, int t,
                                           int32_t* __restrict__ n_full,
                                           int32_t* __restrict__ n_total) {
  const int P = B * group;
  const int p0 = t * KVR_ATTN_QROWS;
  const int p1 = min(P, p0 + KVR_ATTN_QROWS) - 1;
  const int u_min = T[p0 / group], u_max = T[p1 / group];
  n_full[t] = (u_min + 1) / KVR_ATTN_KV_TILE;
  n_total[t] = (u_max + KVR_ATTN_KV_TILE) / KVR_ATTN_KV_TILE;
}

// cos / sin of g * theta^(-2i/d) for packed row r and frequency i, built in
// float64 and stored as a float32 pair of the table [B][d/2].  g is the
// row's global position: gpos[T[r]], or T[r] itself when there is no map.
__device__ __forceinline__ void rope_entry(const int32_t* __restrict__ T,
                                           const int32_t* __restrict__ gpos, int half,
                                           double theta, int idx, float2* __restrict__ tab) {
  const int r = idx / half, i = idx - r * half;
  const double inv = pow(theta, -(2.0 * i) / (2.0 * half));
  const int g = gpos ? gpos[T[r]] : T[r];
  const double ang = static_cast<double>(g) * inv;
  double sn, cs;
  sincos(ang, &sn, &cs);
  tab[idx] = make_float2(static_cast<float>(cs), static_cast<float>(sn));
}

// entry idx of the tables (plan entries first, then the RoPE table)
__device__ __forceinline__ void table_entry(const LayerTables& L, int idx) {
  if (idx < L.n_tiles)
    plan_entry(L.T, L.B, L.group, idx, L.n_full, L.n_total);
  else if (idx - L.n_tiles < L.B * L.half)
    rope_entry(L.T, L.gpos, L.half, L.theta, idx - L.n_tiles, L.tab);
}

}  // namespace kvr
