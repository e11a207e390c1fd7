// Cascade decode for a shared prefix, gfx950: the prefix work-groups.
//
// When every sequence of the batch starts with the same physical blocks (a
// prompt prefix held once with a reference count per user: "01.
// PagedAttention 详解" §6, sharing through the block table), the decode step
// splits into
//   * the prefix part: the query rows of ALL sequences against the one copy
//     of the prefix's K/V. For each kv head this is a dense product of
//     (num_seqs * group) query rows with prefix_len keys, so it runs on the
//     matrix cores (the core of pa_mq.h) and reads the prefix from HBM once
//     instead of once per sequence;
//   * the suffix part: each sequence's own positions past the prefix, as the
//     ordinary decode items;
//   * the combine of both kinds of (max, exp-sum, weighted V) partials, with
//     the split-K algebra of the ordinary path.
// The result is the plain attention of every position < L (an exact
// reformulation, up to fp32 rounding and the 2-byte rounding of the
// softmax weights fed to the matrix cores). The first two parts share one
// launch (cascade_fused_kernel in pa_decode.hip); the combine kernel follows.
//
// This file holds the prefix part as a work-group body. Work-group wg of
// (kv head g, row tile rt, chunk): wg = g + Hkv * (rt + row_tiles * chunk),
// cascade_waves(D) waves of kCascadeRowBlocks 16-row blocks (4 x 1 at both
// head sizes). Rows are (sequence, query head) pairs of kv head g; each row's
// keys end at min(L, prefix_len); the work-group writes one (reference max,
// exp-sum, unnormalised O) partial per row into partial slot `chunk` of the
// workspace. RD: steps of K/V loads in flight (the LDS ring holds RD + 1);
// LEAN: the core's lower-register form (see mq_attend).
#pragma once

#include "pa_device.h"
#include "pa_launch.h"
#include "pa_mq.h"

namespace pa {

template <int D, int RD>
struct PrefixLds {
  int32_t tbl[kPrefixChunk / 16];
  int limit[cascade_waves(D)];
  MqLds<D, RD + 1> mq;
};

template <class DT, int D, int G, int RD, bool LEAN = false>
__device__ __forceinline__ void cascade_prefix_wg(const DecodeParams& a, int wg,
                                                  PrefixLds<D, RD>& sm) {
  constexpr int W = cascade_waves(D);
  constexpr int RB = kCascadeRowBlocks;
  constexpr int NT = W * 64;
  static_assert(D == 64 || D == 128, "head size");
  int32_t* s_tbl = sm.tbl;
  int* s_limit = sm.limit;

  const int Hkv = a.num_kv_heads;
  const int g = wg % Hkv;
  wg /= Hkv;
  const int rt = wg % a.prefix_row_tiles;
  const int chunk = wg / a.prefix_row_tiles;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15;               // this lane's query column
  const int grp = lane >> 4;

  const int R = a.num_seqs * G;          // query rows of kv head g
  const int c0 = chunk * kPrefixChunk;
  const int c1 = min(a.prefix_len, c0 + kPrefixChunk);
  const int lbs = a.log2_block_size;
  const int bs = a.block_size;
  const int b0 = c0 >> lbs;
  const int nb = (c1 - c0 + bs - 1) >> lbs;
  static_assert(kPrefixChunk / 16 <= NT, "one table entry per thread");
  // Row block b of this wave: row rt * rows-per-work-group + wave * 16 * RB +
  // 16 * b + j, a (sequence, query head) pair of kv head g.
  int s[RB], h[RB];
  bool row_ok[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int r = rt * cascade_rows_per_wg(D) + wave * 16 * RB + 16 * b + j;
    row_ok[b] = r < R;
    s[b] = row_ok[b] ? r / G : 0;
    h[b] = g * G + (row_ok[b] ? r % G : 0);
  }
  // The lengths, the queries and the chunk's table entries do not depend on
  // one another, so their loads are in flight together. Row 0 of the tables
  // holds the prefix.
  int len[RB];                           // s[b] = 0 outside the batch: no load is conditional
#pragma unroll
  for (int b = 0; b < RB; ++b) len[b] = a.lens[s[b]];
  u32x4_t qb[RB][D / 32];
#pragma unroll
  for (int b = 0; b < RB; ++b)
    mq_load_q<D, true>(qb[b], a.q + ((int64_t)s[b] * a.num_q_heads + h[b]) * D, row_ok[b],
                       a.scale_log2 < 0.f);
  const int tb = a.bt[b0 + min(tid, nb - 1)];   // nb >= 1: the chunk starts below prefix_len

  int limit[RB];                         // keys each row may use: min(L, prefix_len)
  int wl = 0;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int L = len[b] < 0 ? 0 : (len[b] > a.len_cap ? a.len_cap : len[b]);
    limit[b] = row_ok[b] ? min(L, a.prefix_len) : 0;
    wl = max(wl, limit[b]);
  }
  // The work-group's largest limit: K/V rows at or past it are not positions
  // of any of its sequences (possibly never written), so they are not read.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wl = max(wl, __shfl_xor(wl, o));
  if (lane == 0) s_limit[wave] = wl;
  if (tid < nb) s_tbl[tid] = (uint64_t)(uint32_t)tb < (uint64_t)a.num_blocks ? tb : -1;  // corrupt: skip
  __syncthreads();
  int wg_limit = s_limit[0];
#pragma unroll
  for (int w = 1; w < W; ++w) wg_limit = max(wg_limit, s_limit[w]);
  const int kend = min(c1, wg_limit);

  int row_end[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b)           // rows past the batch attend unmasked with q = 0
    row_end[b] = row_ok[b] ? min(limit[b], c1) : kend;   // and are not written
  MqState<D, RB> st;
  st.init();
  auto blk_of = [&](int t) -> int { return s_tbl[(t >> lbs) - b0]; };
  mq_attend<DT, D, RB, W, RD, LEAN>(st, qb, sm.mq, static_cast<const uint16_t*>(a.kc),
                          static_cast<const uint16_t*>(a.vc), (int64_t)Hkv * D, g, c0, kend,
                          row_end, fabsf(a.scale_log2), bs, blk_of);

  // Partial of this chunk for each row: (reference max, sum of weights,
  // unnormalised O), consistent with one another whatever the reference.
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const float lsum = mq_sum_over_groups(st.lsum[b]);
    if (!row_ok[b]) continue;
    const int64_t pi = ((int64_t)s[b] * a.num_q_heads + h[b]) * a.part_stride + chunk;
    if (grp == 0) {
      a.ws_m[pi] = st.m[b];
      a.ws_l[pi] = lsum;
    }
    float* po = a.ws_o + pi * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt) =
          make_float4(st.acc[b][dt][0], st.acc[b][dt][1], st.acc[b][dt][2], st.acc[b][dt][3]);
  }
}

}  // namespace pa
