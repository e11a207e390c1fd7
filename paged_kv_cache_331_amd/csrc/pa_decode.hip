// Paged decode attention kernels for gfx950 (CDNA4, wave64).
//
// What is computed: for a sequence s and query head h, softmax over the
// logits scale * q . K_t of positions t < L, then the weighted sum of V_t,
// with K_t / V_t reached through the sequence's block table
// ("PagedAttention 机制" §5.3.4 conceptual kernel; "01. PagedAttention 详解"
// §3 layout and §4 decode loop over the table's blocks). Long sequences are
// split into partitions (the book's §4 / §9: v2 uses split-K over long
// sequences) whose partial results a second kernel combines.
//
// Work decomposition (a design for this chip, not taken from the pages):
//  * One work-group (4 waves) per (kv head g, partition p, sequence s). The G
//    query heads that share kv head g are all served by that work-group, so
//    every K/V row is fetched from HBM once per step.
//  * The partition's block-table entries are staged once into LDS; each wave
//    reads the block id of its tile from LDS and makes it wave-uniform.
//  * A wave walks 16-token tiles (8-token tiles for short partitions of a
//    2-byte cache at head size 128). Lanes form "token rows"; each lane holds
//    16 bytes of one token (8 dimensions of a 2-byte cache, 16 of an FP8 one
//    at head size 128), so one load instruction reads whole K or V rows of
//    4, 8 or 16 consecutive slots. Whole rows per instruction and
//    non-temporal loads measured ~15% faster than half rows with ordinary
//    loads for this gather. The q.k partials are summed inside the row with
//    DPP; nothing crosses rows in the loop.
//  * Each token row keeps its own softmax reference / exp-sum / V
//    accumulator (online softmax; the reference moves, with an exact
//    rescale by exp2(m_old - m_new), only when a tile's max exceeds it by
//    more than 8 in log2 units); rows, then waves, are merged once at the
//    end.
//  * Positions >= L inside the last tile are excluded by select: the logit
//    becomes -inf and the V row is replaced by zeros, so whatever those slots
//    hold (even NaN) cannot reach the result. Table entries past the last
//    block are never read.
//  * Write-then-attend (the book's §4 decode phase: the new token's k/v go to
//    the next slot of the last block, then attention covers it too), when
//    the call appends: the item holding position L-1 reads the cached
//    positions before it and takes the new token from k_new / v_new as one
//    more tile, on the wave that would take the next tile; that wave's row-0
//    lanes also store the row at its slot. The slot is never read in the
//    same launch, so the store needs no ordering against any load.
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"
#include "pa_prefix.h"

namespace pa {
namespace {

// Write-then-attend: the new token of sequence s (position app = L - 1) is
// stored at its slot table[app / bs] * bs + app % bs, kv head g's part by
// the first LPR threads (one token row of lanes, DL dimensions each); the
// slot is recorded once per sequence (kv head 0). A table entry outside the
// pool stores nothing, as the separate cache write skips such slots.
template <class KV, int DL, int LPR>
__device__ __forceinline__ void append_row(const DecodeParams& a, int s, int g, int app, int D,
                                           int tid) {
  if (app < 0) {
    if (g == 0 && tid == 0 && a.slots_out) a.slots_out[s] = -1;
    return;
  }
  const int32_t blk = a.bt[(int64_t)s * a.max_blocks_per_seq + (app >> a.log2_block_size)];
  const int32_t slot = blk * a.block_size + (app & (a.block_size - 1));
  if (g == 0 && tid == 0 && a.slots_out) a.slots_out[s] = slot;
  if (tid >= LPR || (uint64_t)(uint32_t)blk >= (uint64_t)a.num_blocks) return;
  const int64_t src = ((int64_t)s * a.num_kv_heads + g) * D + tid * DL;
  const int64_t dst = (int64_t)slot * a.num_kv_heads * D + (int64_t)g * D + tid * DL;
  using elem = typename KV::elem;
  KV::store(const_cast<elem*>(static_cast<const elem*>(a.kc)) + dst,
            KV::from_src(a.k_new + src, a.k_scale_w));
  KV::store(const_cast<elem*>(static_cast<const elem*>(a.vc)) + dst,
            KV::from_src(a.v_new + src, a.v_scale_w));
}

constexpr float kEmptyMax = -1.0e30f;  // running max before any token: finite, so
                                       // exp2(m_old - m_new) never sees inf - inf
constexpr float kSlack = 8.f;              // lazy softmax reference: weights stay <= 2^8
// Tokens per wave iteration: 16, or 8 in the one-work-group-per-item kernel
// for partitions of at most kShortPartition tokens over a 2-byte cache at
// head size 128 (a tile is always at least two load rows). Short items are
// latency-bound; the half tiles measured 50.1-50.8 us against 51.9-53.1 on
// the cascade's suffix items and within noise on short partitions of the
// MHA and GQA batches, and 8-16% slower on long partitions, so only short
// partitions take them.
constexpr int kTileTokens = 16;
constexpr int kShortTileTokens = 8;
constexpr int kShortPartition = 512;
#ifndef PA_LONG_ITEM_TOKENS
#define PA_LONG_ITEM_TOKENS 256
#endif
constexpr int kLongItemTokens = PA_LONG_ITEM_TOKENS;
constexpr int kTableChunk = 256;           // table entries staged per LDS pass

// Exchanges within a token row of 8 or 16 lanes, for reductions where lane c
// pairs with a partner that differs in bit B of c: row_mirror (c <-> 15 - c)
// for bit 3, row_half_mirror (c <-> 7 - c) for bit 2, quad xors for bits 1
// and 0. The mirrors also flip the lower bits, which only reorders lanes
// that hold the same values at that step of the reductions below.
template <int B>
__device__ __forceinline__ float partner(float x) {
  if constexpr (B == 3) return dpp<kDppMirror>(x);
  else if constexpr (B == 2) return dpp<kDppHalfMirror>(x);
  else if constexpr (B == 1) return dpp<kDppQuadXor2>(x);
  else return dpp<kDppQuadXor1>(x);
}

// One reduce-scatter step on bit B over the first N values: the lane keeps
// the half its bit B selects, summed with the partner's copy of that half.
template <int B, int N>
__device__ __forceinline__ void scatter_step(float* v, int col) {
  const bool hi = ((col >> B) & 1) != 0;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float keep = hi ? v[k + N / 2] : v[k];
    const float send = hi ? v[k] : v[k + N / 2];
    v[k] = keep + partner<B>(send);
  }
}

// Reduce-scatter of N partial sums over the 2^LB lanes of a token row: lane
// c ends with the complete sums of values c * N / 2^LB .. (c + 1) * N / 2^LB - 1
// in v[0 ..], where each lane started with its share of every value.
template <int N, int LB>
__device__ __forceinline__ void reduce_scatter(float* v, int col) {
  if constexpr (LB == 4) {
    scatter_step<3, N>(v, col);
    scatter_step<2, N / 2>(v, col);
    scatter_step<1, N / 4>(v, col);
    scatter_step<0, N / 8>(v, col);
  } else {
    scatter_step<2, N>(v, col);
    scatter_step<1, N / 2>(v, col);
    scatter_step<0, N / 4>(v, col);
  }
}

// One all-gather step on bit B: the lane's N words and the partner's N words
// (the neighbouring block) become 2N words in block order.
template <int B, int N>
__device__ __forceinline__ void gather_step(uint32_t* w, int col) {
  const bool hi = ((col >> B) & 1) != 0;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const uint32_t mine = w[k];
    const uint32_t r = __float_as_uint(partner<B>(__uint_as_float(mine)));
    w[k] = hi ? r : mine;
    w[k + N] = hi ? mine : r;
  }
}

// All-gather over bits B0 .. LB-1 of the lane index: each lane starts with the
// W0 words of block c >> B0 (lanes that differ only in bits below B0 hold the
// same block) and ends with all W0 << (LB - B0) words in block order.
template <int W0, int B0, int LB>
__device__ __forceinline__ void all_gather(uint32_t* w, int col) {
  if constexpr (B0 <= 0) gather_step<0, W0>(w, col);
  if constexpr (B0 <= 1) gather_step<1, (W0 << (1 - (B0 < 1 ? B0 : 1)))>(w, col);
  if constexpr (B0 <= 2) gather_step<2, (W0 << (2 - (B0 < 2 ? B0 : 2)))>(w, col);
  if constexpr (LB == 4 && B0 <= 3) gather_step<3, (W0 << (3 - (B0 < 3 ? B0 : 3)))>(w, col);
}

union Vec16 {
  uint4 v;
  uint32_t w[4];
};

template <int D, int G>
struct DecodeLds {
  int32_t tbl[kTableChunk];
  float part[kDecodeWaves][G][D + 2];
};

// The end of an item: each wave has left its per-head (max, exp-sum) in
// part[wave][h][D], part[wave][h][D + 1] and its unnormalised sums in
// part[wave][h][0 .. D-1] (the caller synchronised). The waves are merged by
// rescaling each to the common max; the item writes its output rows
// (finish) or its partials in slot slot_base + p.
template <class DT, int D, int G>
__device__ __forceinline__ void merge_waves(const DecodeParams& a, int s, int g, int p,
                                            bool finish, const float (&part)[kDecodeWaves][G][D + 2],
                                            int tid) {
  using S = Storage<DT>;
  constexpr int NW = kDecodeWaves;
  constexpr int NT = NW * 64;
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D;
    const int d = i % D;
    float M = part[0][h][D];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, part[w][h][D]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = fast_exp2(part[w][h][D] - M);
      num = fmaf(c, part[w][h][d], num);
      den = fmaf(c, part[w][h][D + 1], den);
    }
    num *= a.v_scale;                                   // 1 unless the cache is FP8
    const int64_t oh = (int64_t)s * a.num_q_heads + (int64_t)g * G + h;
    if (finish) {
      a.out[oh * D + d] = S::from_float(den > 0.f ? num / den : 0.f);
    } else {
      const int64_t pi = oh * a.part_stride + a.slot_base + p;
      a.ws_o[pi * D + d] = num;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = den;
      }
    }
  }
}

// One work item: kv head g, sequence s, partition p. Uniform over the
// work-group (every thread takes the same path and the same barriers).
// APP: the call appends each sequence's new token (write-then-attend);
// instantiated separately so that a plain decode carries none of its code.
// TILE: tokens per wave iteration (raised to two load rows if smaller).
template <class DT, class KT, int D, int G, bool APP, int TILE>
__device__ __forceinline__ void decode_item(const DecodeParams& a, int g, int s, int p,
                                            DecodeLds<D, G>& sm) {
  using S = Storage<DT>;
  constexpr int DL = LaneDims<KT, D>::value;   // dimensions held per lane (16 bytes)
  using KV = Kv<DT, KT, DL>;
  using elem = typename KV::elem;
  using row_t = typename KV::row;
  constexpr int NW = kDecodeWaves;
  constexpr int LPR = D / DL;          // lanes per token row
  constexpr int ROWS = 64 / LPR;       // token rows per load instruction
  constexpr int kTile = TILE > 2 * ROWS ? TILE : 2 * ROWS;   // tokens per wave iteration
  constexpr int TG = kTile / ROWS;     // load instructions per tile and tensor
  static_assert(TG % 2 == 0, "p.V pairs rows tg, tg+1");
  constexpr int NT = NW * 64;
  static_assert(D == 64 || D == 128, "head size");

  int32_t* s_tbl = sm.tbl;
  auto& s_part = sm.part;
  const int Hkv = a.num_kv_heads;

  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int start = a.tok_offset + p * a.part_tokens;
  const int tid = threadIdx.x;
  // Position of the appended token, or -1 (nothing appended, or L = 0).
  const int app = APP ? L - 1 : -1;
  if (start >= L) {
    // The first partition of a sequence with no token past the offset stores
    // its appended token (inside a cascade's shared prefix, which callers
    // must not do: the prefix work-groups of the same launch read that block).
    if (APP && p == 0) append_row<KV, DL, LPR>(a, s, g, app, D, tid);
    // An empty sequence's output is zero (a cascade's combine writes it).
    if (p == 0 && !a.always_combine) {
      uint16_t* o = a.out + ((int64_t)s * a.num_q_heads + (int64_t)g * G) * D;
      for (int i = tid; i < G * D; i += NT) o[i] = 0;
    }
    return;
  }
  const int end = min(L, start + a.part_tokens);
  // With an append, the partition holding position L - 1 reads its cached
  // positions [start, L - 1) from the caches and takes the new token from
  // k_new / v_new (after its tiles, below): the slot it stores is never read
  // in this launch, so no ordering between the store and the loads is needed.
  const bool own_app = APP && app >= start && app < end;
  const int end_main = own_app ? app : end;
  // partitions holding tokens; one of them: this item writes the output
  const int np = (L - a.tok_offset + a.part_tokens - 1) / a.part_tokens;
  const bool finish = np == 1 && !a.always_combine;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row = lane / LPR;
  const int col = lane % LPR;
  const int64_t tok_stride = (int64_t)Hkv * D;        // elements between slots
  const int64_t lane_elem = row * tok_stride + (int64_t)g * D + col * DL;
  const elem* kc = static_cast<const elem*>(a.kc);
  const elem* vc = static_cast<const elem*>(a.vc);

  // q slices of the G query heads of this kv head (raw storage words).
  uint32_t qw[G][DL / 2];
  {
    const uint16_t* qs = a.q + ((int64_t)s * a.num_q_heads + (int64_t)g * G) * D + col * DL;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < DL / 8; ++c) {
        Vec16 t;
        t.v = *reinterpret_cast<const uint4*>(qs + h * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) qw[h][4 * c + e] = t.w[e];
      }
  }

  float m[G], l[G], acc[G][DL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kEmptyMax;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < DL; ++d) acc[h][d] = 0.f;
  }

  const int32_t* bt_row = a.bt + (int64_t)s * a.max_blocks_per_seq;
  const int bs = a.block_size;
  const int lbs = a.log2_block_size;
  const int first_blk = start >> lbs;            // start is block aligned
  // one past the last block read (first_blk when only the new token is left)
  const int end_blk = end_main > start ? ((end_main - 1) >> lbs) + 1 : first_blk;
  const float sl2 = a.scale_log2;

  // With at least as many (head, token) logits per tile as lanes in a token
  // row (G * TG >= LPR: grouped heads), the partial dot products are
  // reduce-scattered over the row instead of summed in every lane, so each
  // lane completes J of them, all of one head (hc), and takes their
  // exponentials alone; the packed weights are then gathered back to every
  // lane of the row for p.V. Each lane keeps the running max of its head and
  // a partial exp-sum, merged over the row at the end of the item.
  constexpr int NL = G * TG;
  constexpr bool kScatter = NL >= LPR;
  constexpr int J = kScatter ? NL / LPR : 1;     // logits a lane completes
  constexpr int SH = TG / J;                     // lanes per head in a token row
  constexpr int LB = LPR == 16 ? 4 : 3;          // bits of the lane index within a row
  static_assert(!kScatter || (J <= TG && TG % J == 0 && SH <= 4), "scatter layout");
  float mh = kEmptyMax, lh = 0.f;

  // Online-softmax update of every token row with one 16-token tile whose K/V
  // rows are in kr / vr; positions >= tend are masked out.
  auto attend = [&](const int ts, const int tend, row_t (&kr)[TG], row_t (&vr)[TG]) {
    if constexpr (kScatter) {
      float v[NL];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) v[h * TG + tg] = KV::dot(qw[h], kr[tg], 0.f);
      reduce_scatter<NL, LB>(v, col);
      float lg[J];
#pragma unroll
      for (int j = 0; j < J; ++j) lg[j] = v[j] * sl2;
      if (ts + kTile > tend) {                 // tail tile: mask positions >= tend
#pragma unroll
        for (int j = 0; j < J; ++j)
          lg[j] = ts + ((col * J + j) % TG) * ROWS + row < tend ? lg[j] : -INFINITY;
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
          vr[tg] = ts + tg * ROWS + row < tend ? vr[tg] : KV::zero();
      }
      uint32_t vw[TG][DL / 2];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) KV::pairs(vr[tg], vw[tg]);

      float mx = lg[0];
#pragma unroll
      for (int j = 1; j < J; ++j) mx = fmaxf(mx, lg[j]);
      if constexpr (SH >= 2) mx = fmaxf(mx, dpp<kDppQuadXor1>(mx));
      if constexpr (SH >= 4) mx = fmaxf(mx, dpp<kDppQuadXor2>(mx));
      const bool up = mx > mh + kSlack;
      const float mn = up ? mx : mh;
      const float alpha = up ? fast_exp2(mh - mn) : 1.f;
      mh = mn;
      float pj[J];
#pragma unroll
      for (int j = 0; j < J; ++j) pj[j] = fast_exp2(lg[j] - mn);
      if (__ballot(up) != 0) {                 // uniform: some head moved its reference
        lh *= alpha;
        const int row0 = lane & ~(LPR - 1);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ah = __shfl(alpha, row0 + h * SH);
#pragma unroll
          for (int d = 0; d < DL; ++d) acc[h][d] *= ah;
        }
      }
      // Weights rounded to QT in token pairs (tokens 2i, 2i+1 of a head), and
      // the exp-sum of those rounded weights, counted once per pair.
      uint32_t pw[NL / 2];
      if constexpr (J >= 2) {
#pragma unroll
        for (int k = 0; k < J / 2; ++k) {
          pw[k] = S::pack2(pj[2 * k], pj[2 * k + 1]);
          lh = S::dot2(pw[k], S::kOnes, lh);
        }
        all_gather<J / 2, 0, LB>(pw, col);
      } else {
        const float pn = dpp<kDppQuadXor1>(pj[0]);   // the pair's other token
        const bool odd = (col & 1) != 0;
        pw[0] = odd ? S::pack2(pn, pj[0]) : S::pack2(pj[0], pn);
        const float lt = S::dot2(pw[0], S::kOnes, lh);
        lh = odd ? lh : lt;
        all_gather<1, 1, LB>(pw, col);
      }
#pragma unroll
      for (int i = 0; i < TG / 2; ++i) {
        uint32_t vlo[DL / 2], vhi[DL / 2];
#pragma unroll
        for (int e = 0; e < DL / 2; ++e) {
          vlo[e] = __builtin_amdgcn_perm(vw[2 * i + 1][e], vw[2 * i][e], 0x05040100u);
          vhi[e] = __builtin_amdgcn_perm(vw[2 * i + 1][e], vw[2 * i][e], 0x07060302u);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint32_t pp = pw[h * (TG / 2) + i];
#pragma unroll
          for (int e = 0; e < DL / 2; ++e) {
            acc[h][2 * e] = S::dot2(pp, vlo[e], acc[h][2 * e]);
            acc[h][2 * e + 1] = S::dot2(pp, vhi[e], acc[h][2 * e + 1]);
          }
        }
      }
      return;
    }
    float lg[G][TG];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) lg[h][tg] = row_sum<LPR>(KV::dot(qw[h], kr[tg], 0.f)) * sl2;

    if (ts + kTile > tend) {                   // tail tile: mask positions >= tend
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const bool ok = ts + tg * ROWS + row < tend;
#pragma unroll
        for (int h = 0; h < G; ++h) lg[h][tg] = ok ? lg[h][tg] : -INFINITY;
        vr[tg] = ok ? vr[tg] : KV::zero();
      }
    }
    uint32_t vw[TG][DL / 2];                   // V rows as packed QT pairs
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) KV::pairs(vr[tg], vw[tg]);

    // Online softmax with a lazily moved reference: a row's m only moves
    // when the tile's max exceeds it by more than kSlack (log2 units), so
    // the weights 2^(s - m) stay below 2^kSlack and the accumulators are
    // rescaled only on such tiles -- skipped by the whole wave when no row
    // moved. sum 2^(s-m) v / sum 2^(s-m) does not depend on m.
    float pr[G][TG], alpha[G];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = lg[h][0];
#pragma unroll
      for (int tg = 1; tg < TG; ++tg) mx = fmaxf(mx, lg[h][tg]);
      const bool up = mx > m[h] + kSlack;
      const float mn = up ? mx : m[h];
      alpha[h] = up ? fast_exp2(m[h] - mn) : 1.f;
      moved |= up;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) pr[h][tg] = fast_exp2(lg[h][tg] - mn);
      m[h] = mn;
    }
    if (__ballot(moved) != 0) {                  // uniform
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] *= alpha[h];
#pragma unroll
        for (int d = 0; d < DL; ++d) acc[h][d] *= alpha[h];
      }
    }
    // p.V on v_dot2 over token pairs: the lane's rows tg and tg+1 hold the
    // same DL dimensions of two tokens, so (v_A,d, v_B,d) is one packed word
    // and (p_A, p_B) -- the weights rounded to QT -- another; the exp-sum
    // takes the same rounded weights (a dot2 with (1, 1)).
#pragma unroll
    for (int i = 0; i < TG / 2; ++i) {
      uint32_t vlo[DL / 2], vhi[DL / 2];         // dimension 2e / 2e+1 of tokens A, B
#pragma unroll
      for (int e = 0; e < DL / 2; ++e) {
        vlo[e] = __builtin_amdgcn_perm(vw[2 * i + 1][e], vw[2 * i][e], 0x05040100u);
        vhi[e] = __builtin_amdgcn_perm(vw[2 * i + 1][e], vw[2 * i][e], 0x07060302u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t pp = S::pack2(pr[h][2 * i], pr[h][2 * i + 1]);
        l[h] = S::dot2(pp, S::kOnes, l[h]);
#pragma unroll
        for (int e = 0; e < DL / 2; ++e) {
          acc[h][2 * e] = S::dot2(pp, vlo[e], acc[h][2 * e]);
          acc[h][2 * e + 1] = S::dot2(pp, vhi[e], acc[h][2 * e + 1]);
        }
      }
    }
  };

  // The new token goes to the wave that would take the next tile (tiles are
  // dealt round-robin from wave 0; a table chunk holds a multiple of NW
  // tiles), so it evens out the waves' work instead of adding to it. With a
  // 2-byte cache that wave loads the new rows before its tiles, so their
  // latency hides behind the loop (an FP8 row would hold twice the registers
  // before quantization and is loaded after the loop).
  const int app_wave = ((end_main - start + kTile - 1) / kTile) % NW;
  const bool app_here = own_app && wave == app_wave;   // uniform
  const int64_t app_src = ((int64_t)s * Hkv + g) * D + col * DL;
  constexpr bool kEarlyRows = !std::is_same<KT, Fp8>::value;
  row_t kn_early{}, vn_early{};
  if (kEarlyRows && app_here) {
    kn_early = KV::from_src(a.k_new + app_src, a.k_scale_w);
    vn_early = KV::from_src(a.v_new + app_src, a.v_scale_w);
  }

  for (int cb = first_blk; cb < end_blk; cb += kTableChunk) {
    const int nb = min(kTableChunk, end_blk - cb);
    if (cb != first_blk) __syncthreads();        // previous chunk fully consumed
    for (int i = tid; i < nb; i += NT) s_tbl[i] = bt_row[cb + i];
    __syncthreads();
    const int t0 = cb << lbs;
    const int t1 = min(end_main, (cb + nb) << lbs);
    const int ntiles = (t1 - t0 + kTile - 1) / kTile;

    for (int it = wave; it < ntiles; it += NW) {
      const int ts = t0 + it * kTile;            // first position of the tile
      const int blk = __builtin_amdgcn_readfirstlane(s_tbl[(ts >> lbs) - cb]);
      if ((uint64_t)(uint32_t)blk >= (uint64_t)a.num_blocks) continue;  // corrupt entry: skip
      const int off0 = ts & (bs - 1);            // tile never straddles a block (bs % 16 == 0)
      const int64_t base = ((int64_t)blk * bs + off0) * tok_stride + lane_elem;

      row_t kr[TG], vr[TG];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) kr[tg] = KV::load(kc + base + tg * ROWS * tok_stride);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) vr[tg] = KV::load(vc + base + tg * ROWS * tok_stride);

      attend(ts, end_main, kr, vr);
    }
  }
  if (app_here) {
    // The new token, as a tile whose rows all hold it and whose positions
    // past app are masked: token row 0 takes it into its softmax state, and
    // the row-0 lanes store it at the slot, as the separate cache write does;
    // a table entry outside the pool drops both, as a skipped tile does.
    const int32_t blk = __builtin_amdgcn_readfirstlane(bt_row[app >> lbs]);
    const int32_t slot = blk * bs + (app & (bs - 1));
    if (g == 0 && lane == 0 && a.slots_out) a.slots_out[s] = slot;
    if ((uint64_t)(uint32_t)blk < (uint64_t)a.num_blocks) {
      const row_t kn = kEarlyRows ? kn_early : KV::from_src(a.k_new + app_src, a.k_scale_w);
      const row_t vn = kEarlyRows ? vn_early : KV::from_src(a.v_new + app_src, a.v_scale_w);
      if (row == 0) {
        const int64_t dst = (int64_t)slot * tok_stride + (int64_t)g * D + col * DL;
        KV::store(const_cast<elem*>(kc) + dst, kn);
        KV::store(const_cast<elem*>(vc) + dst, vn);
      }
      row_t kr[TG], vr[TG];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        kr[tg] = kn;
        vr[tg] = vn;
      }
      attend(app, app + 1, kr, vr);
    }
  }

  // Merge the token rows of each wave: the R = 64 / LPR lanes col + LPR * r
  // hold the same dimensions. The max and exp-sum of each head reach every
  // lane (lane swaps for lane bits 5 and 4, a DPP rotate for bit 3). The
  // G x DL rescaled sums are reduce-scattered instead: each step keeps half
  // of the values, adding the partner's copy of that half, and leaves the
  // other half to the partner, so lane (row, col) ends with the totals of
  // values row * n .. row * n + n - 1 (value h * DL + d), n = G * DL / R.
  if constexpr (kScatter) {
    // Per-head state of the token row, as the unreduced path keeps it: the
    // max from the first lane of each head, the exp-sum over its lanes.
    float lsum = lh;
    if constexpr (SH >= 2) lsum += dpp<kDppQuadXor1>(lsum);
    if constexpr (SH >= 4) lsum += dpp<kDppQuadXor2>(lsum);
    const int row0 = lane & ~(LPR - 1);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = __shfl(mh, row0 + h * SH);
      l[h] = __shfl(lsum, row0 + h * SH);
    }
  }
  static_assert(LPR == 8 || LPR == 16, "row lanes");
  constexpr int N = G * DL;
  constexpr int n = LPR == 8 ? N / 8 : N / 4;
  float Mh[G], Lh[G], v[N];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = m[h], y = m[h];
    lane_swap32(x, y);
    float M = fmaxf(x, y);
    x = y = M;
    lane_swap16(x, y);
    M = fmaxf(x, y);
    if (LPR == 8) M = fmaxf(M, dpp<kDppRowRor8>(M));
    const float c = fast_exp2(m[h] - M);
    float lw = l[h] * c;
    x = y = lw;
    lane_swap32(x, y);
    lw = x + y;
    x = y = lw;
    lane_swap16(x, y);
    lw = x + y;
    if (LPR == 8) lw += dpp<kDppRowRor8>(lw);
    Mh[h] = M;
    Lh[h] = lw;
#pragma unroll
    for (int d = 0; d < DL; ++d) v[h * DL + d] = acc[h][d] * c;
  }
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {              // lane bit 5
    lane_swap32(v[i], v[i + N / 2]);
    v[i] += v[i + N / 2];
  }
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {              // lane bit 4
    lane_swap16(v[i], v[i + N / 4]);
    v[i] += v[i + N / 4];
  }
  if constexpr (LPR == 8) {                       // lane bit 3
    const bool hi = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const float keep = hi ? v[i + N / 8] : v[i];
      const float send = hi ? v[i] : v[i + N / 8];
      v[i] = keep + dpp<kDppRowRor8>(send);
    }
  }
#pragma unroll
  for (int i = 0; i < n; ++i) {
    const int idx = row * n + i;
    s_part[wave][idx / DL][col * DL + idx % DL] = v[i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_part[wave][h][D] = Mh[h];
      s_part[wave][h][D + 1] = Lh[h];
    }
  }
  __syncthreads();

  merge_waves<DT, D, G>(a, s, g, p, finish, s_part, tid);
}

// ---------------------------------------------------------------------------
// Matrix-core decode item for head size 128 with G >= 4 query heads per kv
// head. The VALU item above spends most of its issue slots on the dot
// products of the G heads; here they are matrix-core products with the G
// heads as G of the 16 columns:
//   S^T (16 positions x 16 heads)  = K (16 x 128) . Q^T (128 x 16)     (v_mfma_f32_16x16x32)
//   O^T (16 dims x 16 heads)      += V^T (16 x 16) . P^T (16 x 16)     (v_mfma_f32_16x16x16, per dimension tile)
// A wave takes 16-position steps of the item in turn. Each step's K and V
// rows (16 rows of 128 elements each) go from global memory straight into
// the wave's own LDS buffers (global_load_lds_dwordx4 with the non-temporal
// hint), MmaRows::kRing steps ahead, so a wave only waits on its own loads
// (with no step ahead, K is waited for first and V lands while the logits
// and weights are computed). The operands are read as:
//   * K as the A operand: lane l holds position l % 16 and elements
//     32 ks + 8 (l / 16) .. + 7 of slice ks;
//   * V^T as the A operand through the transposing LDS reads, which hand
//     each lane one dimension of the four positions 4 (l / 16) .. + 3 (the
//     lane layouts are in MmaRows).
// The k order of P^T is those four positions, whose logits the lane holds in
// S^T, so no weight crosses lanes. FP8 codes become the query's 2-byte type
// (exactly) as the operands are read. Rows in LDS are swizzled: the 16-byte
// unit u of row T sits at u ^ key(T), which keeps both kinds of reads free
// of bank conflicts. Positions past the item's end, and blocks whose table
// entry is out of range, load a zero chunk and are masked; the online
// softmax is the lazy-reference one of the VALU item, per column.
constexpr int kMmaStep = 16;                     // positions per step

typedef int mma_v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) mma_v2i mma_lds_v2i;
typedef short mma_s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mma_s4 mma_lds_s4;
typedef _Float16 mma_h4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 mma_lds_read8(uint32_t addr) {
  const mma_v2i r = *reinterpret_cast<const mma_lds_v2i*>(mq_lds_ptr(addr));
  return make_uint2((uint32_t)r.x, (uint32_t)r.y);
}
// O^T += A . B with 16x16x16 operands (four values of the 2-byte type).
template <class QT> struct Mma16;
template <> struct Mma16<Fp16> {
  static __device__ __forceinline__ f32x4_t run(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(mma_h4, a),
                                                 __builtin_bit_cast(mma_h4, b), c, 0, 0, 0);
  }
};
template <> struct Mma16<Bf16> {
  static __device__ __forceinline__ f32x4_t run(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mma_s4, a),
                                                     __builtin_bit_cast(mma_s4, b), c, 0, 0, 0);
  }
};

// What differs between an FP8 cache and one in the query's 2-byte type.
template <class QT, class KT> struct MmaRows;

// FP8: 128-byte rows (8 units), two to a 256-byte pass over the banks.
// key: bijective on the 8 rows of each parity (K reads: 16 consecutive rows
// at one unit, two halves), and key >> 1 distinct over the rows of one
// parity among 8 aligned rows (V reads of two 16-lane groups together:
// units 2 dd and 2 dd + 1 of rows 4 q .. 4 q + 7). V^T: ds_read_b64_tr_b8 hands lane j of a 16-lane group
// byte j % 8 of the row addressed by group lane 2 y + j / 8 as its byte y;
// group lane 2 y + h points at position 4 (l/16) + y % 4, dimensions
// 16 (2 dd + y / 4) + 8 h, so one read gives lane j dimension 32 dd + j
// (bytes 0-3) and 32 dd + 16 + j (bytes 4-7) of its four positions.
template <class QT> struct MmaRows<QT, Fp8> {
  static constexpr int kRowBytes = 128;
  static constexpr int kRing = 2;                // steps of loads in flight per wave
  static constexpr int kVReads = 4;              // transposing reads per step (2 tiles each)
  static constexpr int kAppLanes = 8;            // lanes holding a row, 16 bytes each
  static __device__ __forceinline__ int key(int T) { return (((T >> 1) & 3) << 1) | ((T >> 3) & 1); }
  static __device__ __forceinline__ uint32_t k_off(int j, int gq, int ks) {
    return j * 128 + (((2 * ks + (gq >> 1)) ^ key(j)) << 4) + 8 * (gq & 1);
  }
  static __device__ __forceinline__ u32x4_t k_operand(uint32_t addr) {
    const uint2 w = mma_lds_read8(addr);
    return u32x4_t{Fp8Pair<QT>::template get<false>(w.x), Fp8Pair<QT>::template get<true>(w.x),
                   Fp8Pair<QT>::template get<false>(w.y), Fp8Pair<QT>::template get<true>(w.y)};
  }
  static __device__ __forceinline__ uint32_t v_off(int j, int gq, int r) {
    const int y = j >> 1;
    const int T = 4 * gq + (y & 3);
    return T * 128 + (((2 * r + (y >> 2)) ^ key(T)) << 4) + 8 * (j & 1);
  }
  // Dimension tiles 2 r and 2 r + 1.
  static __device__ __forceinline__ void v_operands(uint32_t addr, uint2 (&v)[2]) {
    const mma_v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        reinterpret_cast<mma_lds_v2i*>(mq_lds_ptr(addr)));
    const uint32_t w0 = (uint32_t)t.x, w1 = (uint32_t)t.y;
    v[0] = make_uint2(Fp8Pair<QT>::template get<false>(w0), Fp8Pair<QT>::template get<true>(w0));
    v[1] = make_uint2(Fp8Pair<QT>::template get<false>(w1), Fp8Pair<QT>::template get<true>(w1));
  }
  // This lane's 16 bytes of the new token's K / V row, as the cache stores them.
  static __device__ __forceinline__ u32x4_t app_row(const uint16_t* src, float scale) {
    const typename Kv<QT, Fp8, 16>::row r = Kv<QT, Fp8, 16>::from_src(src, scale);
    return u32x4_t{r[0], r[1], r[2], r[3]};
  }
};

// 2-byte rows: 256 bytes (16 units, one pass over the banks). key:
// bijective on 16 rows (K reads: 16 rows at one unit), and key >> 1
// distinct over 8 aligned rows (V reads of two 16-lane groups together:
// units 2 dt and 2 dt + 1 of rows 4 q .. 4 q + 7).
// V^T: ds_read_b64_tr_b16 hands lane j of a 16-lane group element j % 4 of
// the row addressed by group lane 4 y + j / 4 as its element y; group lane
// 4 y + q points at position 4 (l/16) + y, dimensions 16 dt + 4 q, so lane j
// gets dimension 16 dt + j of its four positions.
template <class QT> struct MmaRows<QT, QT> {
  static constexpr int kRowBytes = 256;
  static constexpr int kRing = 0;                // K first, V behind the logits
  static constexpr int kVReads = 8;
  static constexpr int kAppLanes = 16;
  static __device__ __forceinline__ int key(int T) { return ((T & 7) << 1) | ((T >> 3) & 1); }
  static __device__ __forceinline__ uint32_t k_off(int j, int gq, int ks) {
    return j * 256 + (((4 * ks + gq) ^ key(j)) << 4);
  }
  static __device__ __forceinline__ u32x4_t k_operand(uint32_t addr) { return mq_lds_read16(mq_lds_ptr(addr)); }
  static __device__ __forceinline__ uint32_t v_off(int j, int gq, int r) {
    const int y = j >> 2, q = j & 3;
    const int T = 4 * gq + y;
    return T * 256 + (((2 * r + (q >> 1)) ^ key(T)) << 4) + 8 * (q & 1);
  }
  static __device__ __forceinline__ void v_operands(uint32_t addr, uint2 (&v)[1]) {
    v[0] = mq_lds_read_tr16(mq_lds_ptr(addr));
  }
  static __device__ __forceinline__ u32x4_t app_row(const uint16_t* src, float) {
    return *reinterpret_cast<const u32x4_t*>(src);
  }
};

template <class QT, class KT, int RD>
struct MmaLdsRing {
  static constexpr int kTile = kMmaStep * MmaRows<QT, KT>::kRowBytes;
  static constexpr int kBufs = RD + 1;
  alignas(16) uint8_t k[kDecodeWaves][kBufs][kTile];
  alignas(16) uint8_t v[kDecodeWaves][kBufs][kTile];
};

template <class QT, class KT, int G, int RD = MmaRows<QT, KT>::kRing>
struct MmaLds {
  int32_t tbl[kTableChunk];
  union {
    MmaLdsRing<QT, KT, RD> ring;                 // during the walk
    float part[kDecodeWaves][G][128 + 2];        // after it (behind a barrier)
  };
};

// RD: steps of loads in flight per wave. With RD = 0 a step's K loads are
// waited for first, its logits and weights computed while its V loads
// land, and only then V waited for.
template <class QT, class KT, int G, bool APP, int RD = MmaRows<QT, KT>::kRing>
__device__ __forceinline__ void decode_item_mma(const DecodeParams& a, int g, int s, int p,
                                                MmaLds<QT, KT, G, RD>& sm) {
  using S = Storage<QT>;
  using R = MmaRows<QT, KT>;
  using KV = Kv<QT, KT, std::is_same<KT, Fp8>::value ? 16 : 8>;
  constexpr int D = 128;
  constexpr int NW = kDecodeWaves;
  constexpr int NT = NW * 64;
  constexpr int NB = RD + 1;
  constexpr int TILE = MmaLdsRing<QT, KT, RD>::kTile;
  constexpr int WL = TILE / 1024;                // wave loads per tile
  constexpr int UNITS = R::kRowBytes / 16;
  constexpr int VR = R::kVReads;
  constexpr int VT = 8 / VR;                     // dimension tiles per transposing read
  static_assert(G >= 4 && G <= 16, "heads as matrix columns");
  const int Hkv = a.num_kv_heads;
  const int tid = threadIdx.x;

  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int start = a.tok_offset + p * a.part_tokens;
  const int app = APP ? L - 1 : -1;
  if (start >= L) {
    if (APP && p == 0) append_row<KV, 128 / R::kAppLanes, R::kAppLanes>(a, s, g, app, D, tid);
    if (p == 0 && !a.always_combine) {
      uint16_t* o = a.out + ((int64_t)s * a.num_q_heads + (int64_t)g * G) * D;
      for (int i = tid; i < G * D; i += NT) o[i] = 0;
    }
    return;
  }
  const int end = min(L, start + a.part_tokens);
  const bool own_app = APP && app >= start && app < end;
  const int end_main = own_app ? app : end;
  const int np = (L - a.tok_offset + a.part_tokens - 1) / a.part_tokens;
  const bool finish = np == 1 && !a.always_combine;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15;                     // head column / row of a 16-row operand
  const int gq = lane >> 4;
  const int64_t row_bytes = (int64_t)Hkv * R::kRowBytes;   // bytes between slots
  const uint8_t* kc = static_cast<const uint8_t*>(a.kc) + (int64_t)g * R::kRowBytes;
  const uint8_t* vc = static_cast<const uint8_t*>(a.vc) + (int64_t)g * R::kRowBytes;
  const uint8_t* zero = reinterpret_cast<const uint8_t*>(kMqZeroChunk);

  // Q^T as the B operand: column j = head j of the group (zero past G),
  // slice ks = dimensions 32 ks + 8 gq .. + 7.
  u32x4_t qb[4];
  {
    const bool ok = j < G;
    const uint16_t* qs = a.q + ((int64_t)s * a.num_q_heads + (int64_t)g * G + (ok ? j : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qb[ks] = ok ? *reinterpret_cast<const u32x4_t*>(qs + 32 * ks + 8 * gq) : u32x4_t{0u, 0u, 0u, 0u};
  }

  uint32_t koff[4], voff[VR];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = R::k_off(j, gq, ks);
#pragma unroll
  for (int r = 0; r < VR; ++r) voff[r] = R::v_off(j, gq, r);
  // Loads: wave-load w of a tile fills bytes [1024 w, +1024): this lane's 16
  // bytes are unit lane % UNITS of row (1024 w + 16 lane) / row bytes, which
  // holds source unit (lane % UNITS) ^ key(row). The rows of one wave-load
  // (8 at FP8, 4 at 2 bytes) lie in one block, so its first row's slot is
  // wave-uniform; loff is this lane's byte offset from that row.
  uint32_t loff[WL];
  int lrow[WL];
#pragma unroll
  for (int w = 0; w < WL; ++w) {
    lrow[w] = (1024 * w + 16 * lane) / R::kRowBytes;
    loff[w] = (uint32_t)(lrow[w] - (1024 * w) / R::kRowBytes) * (uint32_t)row_bytes +
              (uint32_t)(((lane % UNITS) ^ R::key(lrow[w])) << 4);
  }

  const uint32_t kr0 = (uint32_t)(uintptr_t)&sm.ring.k[wave][0][0];
  const uint32_t vr0 = (uint32_t)(uintptr_t)&sm.ring.v[wave][0][0];
  const int32_t* bt_row = a.bt + (int64_t)s * a.max_blocks_per_seq;
  const int bs = a.block_size;
  const int lbs = a.log2_block_size;
  const float sl2 = a.scale_log2;

  f32x4_t acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kEmptyMax, lsum = 0.f;

  // Step k of this wave in the staged table chunk at block cb (positions
  // t0 + 16 (wave + NW k) ..) into ring buffer k % NB. A step past the
  // wave's last (k >= mine) loads the zero chunk, so every step issues the
  // same number of loads. Returns whether the step's block entry is bad.
  auto issue = [&](int t0, int cb, int tend, int k, int mine) -> bool {
    const int ts = t0 + kMmaStep * (wave + NW * k);
    const int blk = k < mine ? __builtin_amdgcn_readfirstlane(sm.tbl[min((ts >> lbs) - cb, kTableChunk - 1)]) : -1;
    const bool okb = (uint64_t)(uint32_t)blk < (uint64_t)a.num_blocks;
    const uint32_t buf = (uint32_t)(k % NB) * TILE;
    int64_t row[WL];
    bool ok[WL];
#pragma unroll
    for (int w = 0; w < WL; ++w) {
      const int tw = ts + (1024 * w) / R::kRowBytes;      // the wave-load's first position
      ok[w] = okb && ts + lrow[w] < tend;
      row[w] = ((int64_t)blk * bs + (tw & (bs - 1))) * row_bytes + loff[w];
    }
#pragma unroll
    for (int w = 0; w < WL; ++w)               // all of K first, then V
      mq_lds_load16_nt(ok[w] ? kc + row[w] : zero, kr0 + buf + (uint32_t)w * 1024);
#pragma unroll
    for (int w = 0; w < WL; ++w)
      mq_lds_load16_nt(ok[w] ? vc + row[w] : zero, vr0 + buf + (uint32_t)w * 1024);
    return !okb;
  };

  // One step from ring buffer offset buf: positions ts .. ts + 15, masked at
  // tend. wait_v runs between the weights and the V products.
  auto compute = [&](int ts, int tend, uint32_t buf, bool bad, auto wait_v) {
    const uint32_t kt = kr0 + buf;
    const uint32_t vt = vr0 + buf;
    f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) c = Mma<QT>::run(R::k_operand(kt + koff[ks]), qb[ks], c);
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = ts + 4 * gq + i < tend && !bad ? c[i] * sl2 : -INFINITY;
    float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    // A column's reference moves only for a key above it by more than the
    // slack; unless some lane holds one, the column max across the lane
    // groups is not needed. When one does, its column moves, so the
    // accumulators are rescaled in the same branch.
    float mn = m;
    if (__ballot(mx > m + kSlack) != 0) {      // uniform
      mx = mq_max_over_groups(mx);
      mn = mx > m + kSlack ? mx : m;
      const float alpha = fast_exp2(m - mn);   // 1 where this column did not move
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
    }
    m = mn;
    uint2 pb;
    pb.x = Mma<QT>::pack(fast_exp2(lg[0] - mn), fast_exp2(lg[1] - mn));
    pb.y = Mma<QT>::pack(fast_exp2(lg[2] - mn), fast_exp2(lg[3] - mn));
    lsum = S::dot2(pb.x, S::kOnes, lsum);
    lsum = S::dot2(pb.y, S::kOnes, lsum);
    wait_v();
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      uint2 v[VT];
      R::v_operands(vt + voff[r], v);
#pragma unroll
      for (int e = 0; e < VT; ++e) acc[VT * r + e] = Mma16<QT>::run(v[e], pb, acc[VT * r + e]);
    }
  };

  const int first_blk = start >> lbs;            // start is block aligned
  const int end_blk = end_main > start ? ((end_main - 1) >> lbs) + 1 : first_blk;
  for (int cb = first_blk; cb < end_blk; cb += kTableChunk) {
    const int nb = min(kTableChunk, end_blk - cb);
    if (cb != first_blk) __syncthreads();        // previous chunk fully consumed
    for (int i = tid; i < nb; i += NT) sm.tbl[i] = bt_row[cb + i];
    __syncthreads();
    const int t0 = cb << lbs;
    const int t1 = min(end_main, (cb + nb) << lbs);
    const int nsteps = (t1 - t0 + kMmaStep - 1) / kMmaStep;
    const int mine = nsteps > wave ? (nsteps - wave + NW - 1) / NW : 0;   // uniform
    if (mine == 0) continue;
    if constexpr (RD == 0) {
      for (int k = 0; k < mine; ++k) {
        const bool bad = issue(t0, cb, t1, k, mine);
        mq_wait_loads<WL>();                     // K has landed (V was issued after it)
        compute(t0 + kMmaStep * (wave + NW * k), t1, 0u, bad, [] { mq_wait_loads<0>(); });
      }
    } else {
      bool bad[NB];
#pragma unroll
      for (int r = 0; r < RD; ++r) bad[r] = issue(t0, cb, t1, r, mine);
      for (int k0 = 0; k0 < mine; k0 += NB) {
#pragma unroll
        for (int r = 0; r < NB; ++r) {
          const int k = k0 + r;
          if (k >= mine) break;                  // uniform
          bad[(r + RD) % NB] = issue(t0, cb, t1, k + RD, mine);
          mq_wait_loads<RD * 2 * WL>();          // step k's loads have landed
          compute(t0 + kMmaStep * (wave + NW * k), t1, (uint32_t)r * TILE, bad[r], [] {});
        }
      }
    }
    mq_wait_loads<0>();                          // the ring is free again
  }

  // The new token, in the wave that would take the next step: a step whose
  // row 0 holds its row (as the cache stores it) and whose other rows are
  // zero, masked past app. The row's lanes also store it at the slot.
  const int app_wave = ((end_main - start + kMmaStep - 1) / kMmaStep) % NW;
  if (own_app && wave == app_wave) {             // uniform
    const int32_t blk = __builtin_amdgcn_readfirstlane(bt_row[app >> lbs]);
    const int32_t slot = blk * bs + (app & (bs - 1));
    if (g == 0 && lane == 0 && a.slots_out) a.slots_out[s] = slot;
    if ((uint64_t)(uint32_t)blk < (uint64_t)a.num_blocks) {
      // Every load of this wave has landed and been read: buffer 0 is free.
      mq_lds_u32x4* kz = reinterpret_cast<mq_lds_u32x4*>(mq_lds_ptr(kr0));
      mq_lds_u32x4* vz = reinterpret_cast<mq_lds_u32x4*>(mq_lds_ptr(vr0));
#pragma unroll
      for (int i = 0; i < TILE / 16 / 64; ++i) {
        kz[lane + 64 * i] = u32x4_t{0u, 0u, 0u, 0u};
        vz[lane + 64 * i] = u32x4_t{0u, 0u, 0u, 0u};
      }
      if (lane < R::kAppLanes) {
        // lane u holds elements 128 / kAppLanes * u ..: source unit u of row 0,
        // which sits at unit u ^ key(0) = u
        const int64_t src = ((int64_t)s * Hkv + g) * D + (128 / R::kAppLanes) * lane;
        const u32x4_t kn = R::app_row(a.k_new + src, a.k_scale_w);
        const u32x4_t vn = R::app_row(a.v_new + src, a.v_scale_w);
        const int64_t dst = (int64_t)slot * row_bytes + 16 * lane;
        *reinterpret_cast<u32x4_t*>(const_cast<uint8_t*>(kc) + dst) = kn;
        *reinterpret_cast<u32x4_t*>(const_cast<uint8_t*>(vc) + dst) = vn;
        kz[lane] = kn;
        vz[lane] = vn;
      }
      compute(app, app + 1, 0, false, [] {});    // the wave's LDS accesses stay in order
    }
  }

  // Merge: column j (head j < G) of this wave, its dimensions 16 dt + 4 gq + i.
  const float lh = mq_sum_over_groups(lsum);
  __syncthreads();                               // every wave is done with the ring
  if (j < G) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.part[wave][j][16 * dt + 4 * gq + i] = acc[dt][i];
    if (gq == 0) {
      sm.part[wave][j][D] = m;
      sm.part[wave][j][D + 1] = lh;
    }
  }
  __syncthreads();
  merge_waves<QT, D, G>(a, s, g, p, finish, sm.part, tid);
}

// Whether the matrix-core item serves a (cache type, head size, group):
// grouped heads at head size 128 (FP8 GQA-8B 156 against 168 us for the
// VALU item, bf16 GQA-8B 267 against 269, the long-context batch 172 against
// 174; the cascade's short suffix items keep the VALU item, whose LDS
// footprint lets all of them be resident at once).
template <class KT, int D, int G>
struct UseMmaItem {
  static constexpr bool value = D == 128 && G >= 4;
};

// One work-group per item, in the partition kernel's grid order.
template <class QT, class KT, int G, bool APP>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_mma_kernel(const DecodeParams a) {
  __shared__ MmaLds<QT, KT, G> sm;
  int wg = blockIdx.x;
  const int g = wg % a.num_kv_heads;
  wg /= a.num_kv_heads;
  const int s = a.seq_major ? wg / a.num_parts : wg % a.num_seqs;
  const int p = a.seq_major ? wg % a.num_parts : wg / a.num_seqs;
  decode_item_mma<QT, KT, G, APP>(a, g, s, p, sm);
}

// One work-group per item. Work-groups are numbered kv head fastest. With
// many (sequence, kv head) pairs the partition index comes last: every
// sequence's first partition is dispatched before any second one, and
// partitions past a sequence's end (which exit at once) gather at the end of
// the grid. With few pairs (long contexts) the sequence index comes last, so
// one sequence's partitions run together; each order measured faster in its
// regime.
template <class DT, class KT, int D, int G, bool APP, int TILE>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_partition_kernel(const DecodeParams a) {
  __shared__ DecodeLds<D, G> sm;
  int wg = blockIdx.x;
  const int g = wg % a.num_kv_heads;
  wg /= a.num_kv_heads;
  const int s = a.seq_major ? wg / a.num_parts : wg % a.num_seqs;
  const int p = a.seq_major ? wg % a.num_parts : wg / a.num_seqs;
  if constexpr (TILE < kTileTokens) {
    // Short tiles, but an item of more than kLongItemTokens positions takes
    // full tiles: twice the bytes in flight per wave and half the dependent
    // rounds (512-token partitions of the long-context batch: 191 against
    // 196 us).
    int L = a.lens[s];
    L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
    const int start = a.tok_offset + p * a.part_tokens;
    if (min(L, start + a.part_tokens) - start > kLongItemTokens) {
      decode_item<DT, KT, D, G, APP, kTileTokens>(a, g, s, p, sm);
      return;
    }
  }
  decode_item<DT, KT, D, G, APP, TILE>(a, g, s, p, sm);
}

// Persistent grid: gridDim.x (at most the item count) work-groups walk the
// items in partition-major order (kv head fastest, then sequence). Each
// starts with item blockIdx.x; later items come from the counter half of the
// scheduler word as grid + ticket, so a work-group that drew short items
// takes more of them and none waits on a hardware dispatch slot. The counter
// is trusted only when the word's tag half holds sched_tag; otherwise (the
// first call on a workspace) the items are walked with the fixed stride
// gridDim.x. Every item is taken by exactly one work-group under either
// schedule. The counter always returns to zero: on the counted walk the last
// work-group to finish resets it (every ticket has been drawn by then), and
// the combine kernel writes (tag, 0) after every call, which also arms the
// counter after a fixed-stride walk. One counter serves the whole chip:
// splitting it per XCD (each XCD's work-groups on their own share of the
// items, with or without stealing at the end) measured 3-9% slower.
template <class DT, class KT, int D, int G, bool APP>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_persistent_kernel(const DecodeParams a) {
  constexpr bool kMma = UseMmaItem<KT, D, G>::value;
  __shared__ typename std::conditional<kMma, MmaLds<DT, KT, G>, DecodeLds<D, G>>::type sm;
  __shared__ int s_item[2];
  const int Hkv = a.num_kv_heads;
  const int total = Hkv * a.num_seqs * a.num_parts;
  const uint32_t grid = gridDim.x;                 // <= total (host)
  const bool counted = (uint32_t)*a.sched == a.sched_tag;
  int64_t item = blockIdx.x;
  for (int k = 0; item < total; k ^= 1) {
    const int it = (int)item;
    const int g = it % Hkv;
    const int s = (it / Hkv) % a.num_seqs;
    const int p = it / (Hkv * a.num_seqs);
    if constexpr (kMma)
      decode_item_mma<DT, KT, G, APP>(a, g, s, p, sm);
    else
      decode_item<DT, KT, D, G, APP, kTileTokens>(a, g, s, p, sm);
    if (!counted) {
      // The next item writes its waves' sums into sm.part, which threads of
      // this item may still be reading in the cross-wave merge: an item whose
      // partition holds only the appended token meets no barrier before that
      // write.
      __syncthreads();
      item += grid;
      continue;
    }
    // Double-buffered slot: a thread still reading s_item[k] from the previous
    // round cannot be overtaken, since thread 0 writes s_item[k] again only
    // after the barrier below has been passed by every thread. A ticket past
    // the last item (whatever the counter held) ends the walk.
    if (threadIdx.x == 0) {
      const uint32_t t = (uint32_t)(atomicAdd(a.sched, 1ull << 32) >> 32);
      s_item[k] = t < (uint32_t)total - grid ? (int)(grid + t) : total;
    }
    __syncthreads();
    item = s_item[k];
  }
  // A work-group's last ticket (the one past the end) has been drawn. The
  // grid-th work-group to get here is the last to draw: it returns the
  // counter to zero and re-arms the finish count, so the next call finds
  // (tag, 0) even if this call's combine kernel never runs.
  if (counted && threadIdx.x == 0) {
    if (atomicAdd(a.sched_done, 1u) == grid - 1) {
      atomicExch(a.sched, (unsigned long long)a.sched_tag);
      atomicExch(a.sched_done, 0u);
    }
  }
}

// Split-K combine for the sequences with two or more partitions:
//   out = sum_q 2^(m_q - M) o_q / sum_q 2^(m_q - M) l_q,   M = max_q m_q,
// over the partitions q that hold tokens. One work-group per (sequence,
// query head). Threads own a 16-byte chunk of the output row and a strided
// subset of the partitions, so a long sequence's partials are read with
// every thread's loads in flight at once; the subsets are summed through
// LDS. Sequences with one partition were finished by the partition kernel.
template <class DT, int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(const DecodeParams a) {
  using S = Storage<DT>;
  constexpr int NT = kReduceThreads;
  constexpr int NW = NT / 64;
  constexpr int CH = D / 4;              // 16-byte chunks of one output row
  constexpr int GROUPS = NT / CH;        // partition subsets
  __shared__ float s_max[NW];
  __shared__ float s_sum[NT][5];

  const int h = blockIdx.x % a.num_q_heads;
  const int s = blockIdx.x / a.num_q_heads;
  const int tid = threadIdx.x;
  // The partition kernel has finished (stream order): leave the scheduler
  // state the next persistent launch on this workspace expects.
  if (a.sched != nullptr && blockIdx.x == 0 && tid == 0) {
    *a.sched = a.sched_tag;
    *a.sched_done = 0u;
  }
  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int64_t oh = (int64_t)s * a.num_q_heads + h;
  if (L == 0) {                          // a cascade leaves empty sequences to this kernel
    if (a.always_combine)
      for (int d = tid; d < D; d += NT) a.out[oh * D + d] = 0;
    return;
  }
  const int own = L > a.tok_offset ? (L - a.tok_offset + a.part_tokens - 1) / a.part_tokens : 0;
  const int np = a.slot_base + own;      // partial slots holding this sequence's tokens
  if (own <= 1 && !a.always_combine) return;   // finished by the partition kernel

  const float* pm = a.ws_m + oh * a.part_stride;
  const float* pl = a.ws_l + oh * a.part_stride;

  // M = max over the partitions' running maxima.
  float M = kEmptyMax;
  for (int q = tid; q < np; q += NT) M = fmaxf(M, pm[q]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) s_max[tid >> 6] = M;
  __syncthreads();
  M = s_max[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, s_max[w]);

  const int c = tid % CH;
  const int grp = tid / CH;
  const float4* po = reinterpret_cast<const float4*>(a.ws_o + oh * a.part_stride * D) + c;
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int q = grp; q < np; q += GROUPS) {
    const float w = fast_exp2(pm[q] - M);
    const float4 o = po[(int64_t)q * CH];
    den = fmaf(w, pl[q], den);
    acc.x = fmaf(w, o.x, acc.x);
    acc.y = fmaf(w, o.y, acc.y);
    acc.z = fmaf(w, o.z, acc.z);
    acc.w = fmaf(w, o.w, acc.w);
  }
  float* r = s_sum[tid];
  r[0] = den;
  r[1] = acc.x;
  r[2] = acc.y;
  r[3] = acc.z;
  r[4] = acc.w;
  __syncthreads();
  if (grp != 0) return;
  float t[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < GROUPS; ++k) {
#pragma unroll
    for (int e = 0; e < 5; ++e) t[e] += s_sum[k * CH + c][e];
  }
  const float inv = 1.f / t[0];
  uint2 packed;
  packed.x = (uint32_t)S::from_float(t[1] * inv) | ((uint32_t)S::from_float(t[2] * inv) << 16);
  packed.y = (uint32_t)S::from_float(t[3] * inv) | ((uint32_t)S::from_float(t[4] * inv) << 16);
  *reinterpret_cast<uint2*>(a.out + oh * D + c * 4) = packed;
}

// The same combine for calls with few partial slots per row (at most
// kFewParts): each thread owns one 16-byte chunk of one query head's output
// row and walks that row's partials itself, so a work-group covers 256 / (D/4)
// heads of a sequence with no LDS and no barrier. Kernel trace on the
// GQA-8B batch (4 partitions): 5.2 us against 9.9 us for the
// partition-parallel kernel.
constexpr int kFewParts = 16;

template <class DT, int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_few_kernel(const DecodeParams a) {
  using S = Storage<DT>;
  constexpr int CH = D / 4;                        // 16-byte chunks of one output row
  constexpr int HPW = kReduceThreads / CH;         // query heads per work-group
  const int tid = threadIdx.x;
  if (a.sched != nullptr && blockIdx.x == 0 && tid == 0) {
    *a.sched = a.sched_tag;
    *a.sched_done = 0u;
  }
  const int hgroups = (a.num_q_heads + HPW - 1) / HPW;
  const int s = blockIdx.x / hgroups;
  const int h = (blockIdx.x % hgroups) * HPW + tid / CH;
  const int c = tid % CH;
  if (h >= a.num_q_heads) return;
  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int64_t oh = (int64_t)s * a.num_q_heads + h;
  uint2* o = reinterpret_cast<uint2*>(a.out + oh * D) + c;
  if (L == 0) {                                    // a cascade leaves empty sequences here
    if (a.always_combine) *o = make_uint2(0u, 0u);
    return;
  }
  const int own = L > a.tok_offset ? (L - a.tok_offset + a.part_tokens - 1) / a.part_tokens : 0;
  const int np = a.slot_base + own;
  if (own <= 1 && !a.always_combine) return;       // finished by the partition kernel

  const float* pm = a.ws_m + oh * a.part_stride;
  const float* pl = a.ws_l + oh * a.part_stride;
  const float4* po = reinterpret_cast<const float4*>(a.ws_o + oh * a.part_stride * D) + c;
  // Every partial's loads are issued before any is used (np <= kFewParts).
  float mv[kFewParts], lv[kFewParts];
  float4 ov[kFewParts];
#pragma unroll
  for (int q = 0; q < kFewParts; ++q) {
    if (q < np) {
      mv[q] = pm[q];
      lv[q] = pl[q];
      ov[q] = po[(int64_t)q * CH];
    }
  }
  float M = kEmptyMax;
#pragma unroll
  for (int q = 0; q < kFewParts; ++q)
    if (q < np) M = fmaxf(M, mv[q]);
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < kFewParts; ++q) {
    if (q < np) {
      const float w = fast_exp2(mv[q] - M);
      den = fmaf(w, lv[q], den);
      acc.x = fmaf(w, ov[q].x, acc.x);
      acc.y = fmaf(w, ov[q].y, acc.y);
      acc.z = fmaf(w, ov[q].z, acc.z);
      acc.w = fmaf(w, ov[q].w, acc.w);
    }
  }
  const float inv = 1.f / den;
  uint2 packed;
  packed.x = (uint32_t)S::from_float(acc.x * inv) | ((uint32_t)S::from_float(acc.y * inv) << 16);
  packed.y = (uint32_t)S::from_float(acc.z * inv) | ((uint32_t)S::from_float(acc.w * inv) << 16);
  *o = packed;
}

// Cascade decode in one launch. Work-groups [0, items) are the suffix items
// (kv head fastest, then sequence, then partition), the rest the prefix
// work-groups of pa_prefix.h. Every item writes partials, which the combine
// kernel that follows merges with the prefix partials, so no work-group
// waits on another: the prefix work-groups take the slots that the shortest
// suffix items leave, and run while the longest ones still read. The launch
// holds the larger of the two LDS footprints; the prefix work-groups keep
// kFusedPrefixRing steps of loads in flight so that the suffix items keep
// four work-groups per CU (two at G = 8, whose items need the registers).
template <int G> struct FusedWavesPerEu { static constexpr int value = G <= 4 ? 4 : 2; };
template <class DT, int D, int G, bool APP, int TILE>
__global__ __launch_bounds__(kDecodeWaves * 64, FusedWavesPerEu<G>::value) void cascade_fused_kernel(
    const DecodeParams a) {
  static_assert(cascade_waves(D) == kDecodeWaves, "one work-group shape for both kinds");
  // The suffix items: the matrix-core item without a ring (one buffer, 33 KB
  // with the table, so that all suffix items of the prefix-shared batch stay
  // resident: 42.2-42.8 against 42.8-43.1 us for the VALU item) for grouped
  // heads at head size 128, else the VALU item.
  constexpr bool kMma = UseMmaItem<DT, D, G>::value;
  using SuffixLds =
      typename std::conditional<kMma, MmaLds<DT, DT, G, 0>, DecodeLds<D, G>>::type;
  __shared__ union {
    SuffixLds dec;
    PrefixLds<D, kFusedPrefixRing> pre;
  } sm;
  const int Hkv = a.num_kv_heads;
  const int items = Hkv * a.num_seqs * a.num_parts;
  int wg = blockIdx.x;
  if (wg >= items) {
    cascade_prefix_wg<DT, D, G, kFusedPrefixRing, true>(a, wg - items, sm.pre);
    return;
  }
  const int g = wg % Hkv;
  wg /= Hkv;
  if constexpr (kMma)
    decode_item_mma<DT, DT, G, APP, 0>(a, g, wg % a.num_seqs, wg / a.num_seqs, sm.dec);
  else
    decode_item<DT, DT, D, G, APP, TILE>(a, g, wg % a.num_seqs, wg / a.num_seqs, sm.dec);
}

template <class DT, int D>
hipError_t launch_combine(const DecodeParams& a, hipStream_t st) {
  if (a.slot_base + a.num_parts <= kFewParts) {
    constexpr int HPW = kReduceThreads / (D / 4);
    const uint64_t nr = (uint64_t)a.num_seqs * ((a.num_q_heads + HPW - 1) / HPW);
    hipLaunchKernelGGL((decode_reduce_few_kernel<DT, D>), dim3((uint32_t)nr),
                       dim3(kReduceThreads), 0, st, a);
  } else {
    const uint64_t nr = (uint64_t)a.num_q_heads * a.num_seqs;
    hipLaunchKernelGGL((decode_reduce_kernel<DT, D>), dim3((uint32_t)nr), dim3(kReduceThreads),
                       0, st, a);
  }
  return hipGetLastError();
}

template <class DT, class KT, int D, int G, bool APP>
hipError_t launch_dga(const DecodeParams& a, hipStream_t st) {
  const uint64_t nwg = (uint64_t)a.num_kv_heads * a.num_parts * a.num_seqs;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffull) return hipErrorInvalidConfiguration;
  const bool combine = a.num_parts > 1 || a.always_combine;
  if (a.sched != nullptr && combine && a.persist_grid > 0) {
    const uint32_t grid = (uint32_t)(nwg < (uint64_t)a.persist_grid ? nwg : a.persist_grid);
    hipLaunchKernelGGL((decode_persistent_kernel<DT, KT, D, G, APP>), dim3(grid),
                       dim3(kDecodeWaves * 64), 0, st, a);
  } else {
    DecodeParams b = a;
    b.sched = nullptr;                   // the combine leaves the scheduler words alone
    if constexpr (UseMmaItem<KT, D, G>::value) {
      hipLaunchKernelGGL((decode_mma_kernel<DT, KT, G, APP>), dim3((uint32_t)nwg),
                         dim3(kDecodeWaves * 64), 0, st, b);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || !combine) return e;
      return launch_combine<DT, D>(b, st);
    }
    bool short_tiles = false;
    if constexpr (D == 128 && std::is_same<KT, DT>::value)
      short_tiles = a.part_tokens <= kShortPartition;
    if (short_tiles) {
      if constexpr (D == 128 && std::is_same<KT, DT>::value)
        hipLaunchKernelGGL((decode_partition_kernel<DT, KT, D, G, APP, kShortTileTokens>),
                           dim3((uint32_t)nwg), dim3(kDecodeWaves * 64), 0, st, b);
    } else {
      hipLaunchKernelGGL((decode_partition_kernel<DT, KT, D, G, APP, kTileTokens>),
                         dim3((uint32_t)nwg), dim3(kDecodeWaves * 64), 0, st, b);
    }
    if (!combine) return hipGetLastError();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine<DT, D>(b, st);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine<DT, D>(a, st);
}

template <class DT, class KT, int D, int G>
hipError_t launch_dg(const DecodeParams& a, hipStream_t st) {
  return a.k_new != nullptr ? launch_dga<DT, KT, D, G, true>(a, st)
                            : launch_dga<DT, KT, D, G, false>(a, st);
}

template <class DT, class KT, int D>
hipError_t launch_d(const DecodeParams& a, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_dg<DT, KT, D, 1>(a, st);
    case 2: return launch_dg<DT, KT, D, 2>(a, st);
    case 4: return launch_dg<DT, KT, D, 4>(a, st);
    case 8: return launch_dg<DT, KT, D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <class DT, class KT>
hipError_t launch_t(const DecodeParams& a, int head_size, int group, hipStream_t st) {
  switch (head_size) {
    case 64: return launch_d<DT, KT, 64>(a, group, st);
    case 128: return launch_d<DT, KT, 128>(a, group, st);
    default: return hipErrorInvalidValue;
  }
}

template <class DT, int D, int G, bool APP>
hipError_t launch_fused(const DecodeParams& a, hipStream_t st) {
  const uint64_t items = (uint64_t)a.num_kv_heads * a.num_parts * a.num_seqs;
  const uint64_t pre = (uint64_t)a.num_kv_heads * a.prefix_row_tiles * a.prefix_chunks;
  if (items + pre == 0) return hipSuccess;
  if (items + pre > 0x7fffffffull) return hipErrorInvalidConfiguration;
  DecodeParams b = a;
  b.sched = nullptr;                     // not a persistent launch: the words stay as they are
  if constexpr (D == 128) {
    if (a.part_tokens <= kShortPartition) {
      hipLaunchKernelGGL((cascade_fused_kernel<DT, D, G, APP, kShortTileTokens>),
                         dim3((uint32_t)(items + pre)), dim3(kDecodeWaves * 64), 0, st, b);
      const hipError_t e = hipGetLastError();
      return e != hipSuccess ? e : launch_combine<DT, D>(b, st);
    }
  }
  hipLaunchKernelGGL((cascade_fused_kernel<DT, D, G, APP, kTileTokens>),
                     dim3((uint32_t)(items + pre)), dim3(kDecodeWaves * 64), 0, st, b);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_combine<DT, D>(b, st);
}

template <class DT, int D, int G>
hipError_t launch_fused_a(const DecodeParams& a, hipStream_t st) {
  return a.k_new != nullptr ? launch_fused<DT, D, G, true>(a, st)
                            : launch_fused<DT, D, G, false>(a, st);
}

template <class DT, int D>
hipError_t launch_fused_g(const DecodeParams& a, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_fused_a<DT, D, 1>(a, st);
    case 2: return launch_fused_a<DT, D, 2>(a, st);
    case 4: return launch_fused_a<DT, D, 4>(a, st);
    case 8: return launch_fused_a<DT, D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <class DT>
hipError_t launch_fused_d(const DecodeParams& a, int head_size, int group, hipStream_t st) {
  switch (head_size) {
    case 64: return launch_fused_g<DT, 64>(a, group, st);
    case 128: return launch_fused_g<DT, 128>(a, group, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_cascade(const DecodeParams& a, int dtype, int head_size, int group,
                          hipStream_t stream) {
  if (!a.always_combine) return hipErrorInvalidValue;
  return dtype == 0 ? launch_fused_d<Fp16>(a, head_size, group, stream)
                    : launch_fused_d<Bf16>(a, head_size, group, stream);
}

hipError_t launch_decode(const DecodeParams& a, int dtype, bool fp8_cache, int head_size,
                         int group, hipStream_t stream) {
  if (fp8_cache)
    return dtype == 0 ? launch_t<Fp16, Fp8>(a, head_size, group, stream)
                      : launch_t<Bf16, Fp8>(a, head_size, group, stream);
  return dtype == 0 ? launch_t<Fp16, Fp16>(a, head_size, group, stream)
                    : launch_t<Bf16, Bf16>(a, head_size, group, stream);
}

}  // namespace pa
