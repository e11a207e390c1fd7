// Paged prefill for gfx950: the new tokens of each sequence (a whole prompt,
// or a later chunk of one) attend causally to every cached position up to
// their own, through the sequence's block table ("01. PagedAttention 详解"
// §4, prefill phase: the N new tokens' K and V are written into the blocks
// the table points to, then attention runs over them).
//
// Sequence s holds L = context_lens[s] positions after the write; its n new
// tokens are rows query_start[s] .. query_start[s+1]-1 of q / out, at
// positions L - n .. L - 1. The token at position p attends to 0 .. p.
//
// Work decomposition: one work-group per (kv head g, sequence s, tile of
// 128 / G new tokens): its 128 query rows (4 waves x 2 blocks of 16) are
// those tokens' G query heads of kv head g, so each K/V row staged serves
// every row, on the matrix-core core of pa_mq.h. The work-group walks
// positions 0 .. (its last token's position) in chunks of 256 table entries
// staged in LDS; each row masks the keys past its own position. Work items
// with more keys are dispatched first (see the dispatch order below).
#include "pa_launch.h"
#include "pa_mq.h"

namespace pa {
namespace {

constexpr int kSlotThreads = 256;
constexpr int kTblChunk = 256;           // table entries staged per LDS pass
#ifndef PA_PREFILL_ROW_BLOCKS
#define PA_PREFILL_ROW_BLOCKS 2
#endif
constexpr int kPrefillRowBlocks = PA_PREFILL_ROW_BLOCKS;   // 16-row blocks per wave
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
// Waves per work-group at head size 128 (at 64 the 4 KB K tile is four 1 KB
// wave loads: 4 waves). Four waves of two row blocks leave room for two
// work-groups per CU, whose barriers do not hold each other up.
template <int D> struct PrefillWaves { static constexpr int value = D == 128 ? PA_PREFILL_WAVES : 4; };
template <int D>
constexpr int prefill_rows_per_wg() {
  return PrefillWaves<D>::value * kMqRowsPerBlock * kPrefillRowBlocks;
}

// Dispatch order. A work item (sequence s, tile qt) walks c + min(n, (qt + 1)
// TPW) keys, c being the positions cached before its n new tokens, so in a
// chunked prefill the tiles of sequences with long contexts are the longest
// whatever their qt. Each work-group therefore ranks the items by that key
// count (descending, ties by sequence) and takes the item of its own rank;
// the count of items ahead of one is a sum over sequences, since a
// sequence's tiles have the key counts c + TPW, c + 2 TPW, ..., c + n. The
// ranking costs each work-group (items / threads) x sequences steps, so it
// is used up to kByKeysMaxSeqs sequences and kByKeysMaxWork items x
// sequences; beyond that, tiles go by qt, later tiles first (the longest
// order for whole prompts).
#ifndef PA_PREFILL_BY_KEYS_MAX_SEQS
#define PA_PREFILL_BY_KEYS_MAX_SEQS 64
#endif
constexpr int kByKeysMaxSeqs = PA_PREFILL_BY_KEYS_MAX_SEQS;
constexpr int64_t kByKeysMaxWork = 65536;
__device__ __forceinline__ bool by_keys(int num_seqs, int num_tiles) {
  return num_seqs <= kByKeysMaxSeqs &&
         (int64_t)num_seqs * num_seqs * num_tiles <= kByKeysMaxWork;
}

// Clamped view of sequence s's new-token rows: [a, a + n).
__device__ __forceinline__ void new_rows(const PrefillParams& p, int s, int L, int& a, int& n) {
  const int T = p.num_tokens;
  int q0 = p.query_start[s], q1 = p.query_start[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > T ? T : q0);
  q1 = q1 < q0 ? q0 : (q1 > T ? T : q1);
  a = q0;
  n = min(q1 - q0, min(L, p.max_query_len));
}

__global__ __launch_bounds__(kSlotThreads) void prefill_slot_kernel(const PrefillParams p) {
  const int s = blockIdx.y;
  int L = p.lens[s];
  L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
  int a, n;
  new_rows(p, s, L, a, n);
  const int i = blockIdx.x * kSlotThreads + threadIdx.x;
  if (i >= n) return;
  const int pos = L - n + i;
  const int32_t* row = p.bt + (int64_t)s * p.max_blocks_per_seq;
  p.slots[a + i] = row[pos / p.block_size] * p.block_size + pos % p.block_size;
}

// Grouped heads run three work-groups per CU, with the core's lean form (V
// fragments read just before their products) and a register cap that spills
// a few values: chunked GQA prefill 177-179 against 184-188 us. One query
// head per kv head keeps two per CU (the same form measured 93-95 against
// 92-93 us on the MHA prompts). Over an FP8 cache the codes staged in
// registers take the room of the third work-group: two per CU.
template <int G, bool F8> struct PrefillOccupancy {
  static constexpr bool kLean = G >= 4;
  static constexpr int kWavesPerEu = G >= 4 && !F8 ? 3 : 1;   // 1: no bound (two fit)
};

template <class DT, int D, int G, bool F8>
__global__ __launch_bounds__(PrefillWaves<D>::value * 64, (PrefillOccupancy<G, F8>::kWavesPerEu))
void prefill_kernel(const PrefillParams p) {
  using S = Storage<DT>;
  constexpr int W = PrefillWaves<D>::value;
  constexpr int NT = W * 64;
  constexpr int RB = kPrefillRowBlocks;
  constexpr int TPW = prefill_rows_per_wg<D>() / G;   // new tokens per work-group
  static_assert(D == 64 || D == 128, "head size");
  __shared__ int32_t s_tbl[kTblChunk];
  __shared__ int32_t s_seq[3][kByKeysMaxSeqs > 0 ? kByKeysMaxSeqs : 1];   // c, n, a per sequence
  __shared__ int32_t s_item;
  __shared__ MqLds<D, F8 ? 2 : kMqBufs> lds;

  const int Hkv = p.num_kv_heads;
  const int tid = threadIdx.x;
  const int g = blockIdx.x % Hkv;
  const int rank = blockIdx.x / Hkv;
  int s, qt, L, a, n;
  if (by_keys(p.num_seqs, p.num_tiles)) {
    const int S = p.num_seqs;                          // <= kByKeysMaxSeqs
    int cached = 0;
    for (int i = tid; i < S; i += NT) {
      int Li = p.lens[i];
      Li = Li < 0 ? 0 : (Li > p.len_cap ? p.len_cap : Li);
      int ai, ni;
      new_rows(p, i, Li, ai, ni);
      s_seq[0][i] = Li - ni;
      s_seq[1][i] = ni;
      s_seq[2][i] = ai;
      cached |= Li > ni;
    }
    if (tid == 0) s_item = rank < S * p.num_tiles ? rank % S + S * (p.num_tiles - 1 - rank / S) : -1;
    // Whole prompts only (no cached positions): the tile order, later tiles
    // first, is the order by key count but for each sequence's last, partial
    // tile, so the ranking is skipped.
    if (__syncthreads_or(cached)) {
      if (tid == 0) s_item = -1;
      __syncthreads();
      for (int idx = tid; idx < S * p.num_tiles; idx += NT) {
        const int si = idx % S, qi = idx / S;
        const int ni = s_seq[1][si];
        if (qi * TPW >= ni) continue;                  // no token in this tile
        const int x = s_seq[0][si] + min(ni, (qi + 1) * TPW);
        int ahead = 0;
        for (int u = 0; u < S; ++u) {
          const int d = x - s_seq[0][u], nu = s_seq[1][u];
          // tiles of u with more keys: those from qt = d / TPW on
          if (d < nu) ahead += (nu + TPW - 1) / TPW - (d < 0 ? 0 : d / TPW);
          // u's tile with exactly x keys, if any, goes first when u < si
          if (u < si && d > 0 && d <= nu && (d % TPW == 0 || d == nu)) ++ahead;
        }
        if (ahead == rank) s_item = idx;
      }
      __syncthreads();
    }
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item < 0) return;                              // uniform: ranks past the last item
    s = item % S;
    qt = item / S;
    n = __builtin_amdgcn_readfirstlane(s_seq[1][s]);
    if (qt * TPW >= n) return;                         // uniform: no token in this tile
    L = __builtin_amdgcn_readfirstlane(s_seq[0][s]) + n;
    a = __builtin_amdgcn_readfirstlane(s_seq[2][s]);
  } else {
    s = rank % p.num_seqs;
    qt = p.num_tiles - 1 - rank / p.num_seqs;         // later tiles first
    L = p.lens[s];
    L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
    new_rows(p, s, L, a, n);
    if (qt * TPW >= n) return;                         // uniform: no token in this tile
  }

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15;
  const int grp = lane >> 4;
  const int kend = L - n + min(n, (qt + 1) * TPW);     // one past the tile's last position

  // Row block b of this wave: work-group rows wave*16*RB + 16*b + j, each a
  // (new token, query head of kv head g) pair. Rows past the sequence's new
  // tokens attend unmasked with q = 0 and are not written.
  int ti[RB], h[RB], row_end[RB];
  bool row_ok[RB];
  u32x4_t qb[RB][D / 32];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int r = wave * kMqRowsPerBlock * RB + kMqRowsPerBlock * b + j;
    ti[b] = qt * TPW + r / G;                          // new token index in the sequence
    h[b] = g * G + r % G;
    row_ok[b] = ti[b] < n;
    row_end[b] = row_ok[b] ? L - n + ti[b] + 1 : kend; // causal: keys 0 .. its position
    mq_load_q<D>(qb[b], p.q + ((int64_t)(a + (row_ok[b] ? ti[b] : 0)) * p.num_q_heads + h[b]) * D,
                 row_ok[b], p.scale_log2 < 0.f);
  }
  MqState<D, RB> st;
  st.init();

  const int32_t* bt_row = p.bt + (int64_t)s * p.max_blocks_per_seq;
  const int lbs = p.log2_block_size;
  const int bs = p.block_size;
  const int64_t tok_stride = (int64_t)Hkv * D;
  const int chunk_tokens = kTblChunk * bs;
  for (int c0 = 0; c0 < kend; c0 += chunk_tokens) {
    const int c1 = min(kend, c0 + chunk_tokens);
    const int b0 = c0 >> lbs;
    const int nb = (c1 - c0 + bs - 1) >> lbs;
    for (int i = tid; i < nb; i += NT) {
      const int blk = bt_row[b0 + i];
      s_tbl[i] = (uint64_t)(uint32_t)blk < (uint64_t)p.num_blocks ? blk : -1;
    }
    __syncthreads();
    auto blk_of = [&](int t) -> int { return s_tbl[(t >> lbs) - b0]; };
    mq_attend<DT, D, RB, W, F8 ? 1 : kMqRing, PrefillOccupancy<G, F8>::kLean, F8>(
        st, qb, lds, p.kc, p.vc, tok_stride, g, c0, c1, row_end, fabsf(p.scale_log2), bs,
        blk_of);   // ends with a barrier: s_tbl is free again
  }

#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const float lsum = mq_sum_over_groups(st.lsum[b]);
    if (!row_ok[b]) continue;
    const float inv = F8 ? p.v_scale / lsum : 1.f / lsum;
    uint16_t* o = p.out + ((int64_t)(a + ti[b]) * p.num_q_heads + h[b]) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      uint2 w;
      w.x = (uint32_t)S::from_float(st.acc[b][dt][0] * inv) |
            ((uint32_t)S::from_float(st.acc[b][dt][1] * inv) << 16);
      w.y = (uint32_t)S::from_float(st.acc[b][dt][2] * inv) |
            ((uint32_t)S::from_float(st.acc[b][dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(o + 16 * dt) = w;
    }
  }
}

template <class DT, int D, int G, bool F8>
hipError_t launch_pf(const PrefillParams& p, hipStream_t st) {
  constexpr int TPW = prefill_rows_per_wg<D>() / G;
  PrefillParams q = p;
  q.num_tiles = (p.max_query_len + TPW - 1) / TPW;
  const uint64_t nwg = (uint64_t)p.num_kv_heads * p.num_seqs * q.num_tiles;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffull) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<DT, D, G, F8>), dim3((uint32_t)nwg),
                     dim3(PrefillWaves<D>::value * 64), 0, st,
                     q);
  return hipGetLastError();
}

template <class DT, int D, bool F8>
hipError_t launch_pf_g(const PrefillParams& p, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_pf<DT, D, 1, F8>(p, st);
    case 2: return launch_pf<DT, D, 2, F8>(p, st);
    case 4: return launch_pf<DT, D, 4, F8>(p, st);
    case 8: return launch_pf<DT, D, 8, F8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <class DT, bool F8>
hipError_t launch_pf_d(const PrefillParams& p, int head_size, int group, hipStream_t st) {
  switch (head_size) {
    case 64: return launch_pf_g<DT, 64, F8>(p, group, st);
    case 128: return launch_pf_g<DT, 128, F8>(p, group, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_size, int group, bool fp8,
                          hipStream_t stream) {
  if (fp8)
    return dtype == 0 ? launch_pf_d<Fp16, true>(p, head_size, group, stream)
                      : launch_pf_d<Bf16, true>(p, head_size, group, stream);
  return dtype == 0 ? launch_pf_d<Fp16, false>(p, head_size, group, stream)
                    : launch_pf_d<Bf16, false>(p, head_size, group, stream);
}

hipError_t launch_prefill_slots(const PrefillParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_query_len == 0) return hipSuccess;
  const dim3 grid((p.max_query_len + kSlotThreads - 1) / kSlotThreads, p.num_seqs);
  hipLaunchKernelGGL(prefill_slot_kernel, grid, dim3(kSlotThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
