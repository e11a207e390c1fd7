// Multi-query paged attention core on the gfx950 matrix cores: many query rows
// that share a kv head, attended to a range of positions reached through a
// block table. Used by the cascade's shared-prefix kernel and by prefill.
//
// A work-group is W wave64s (4 by default); each wave owns RB blocks of 16
// query rows. With
// v_mfma_f32_16x16x32 (lane l: A row l%16, B column l%16, k = 8*(l/16)..+7;
// C column l%16, rows 4*(l/16)..+3) one 32-key step computes, per row block,
//   S^T(16 keys x 16 queries)   = K(16 keys x D) . Q^T(D x 16 queries)   (two key tiles)
//   O^T(16 dims x 16 queries)  += V^T(16 dims x 32 keys) . P^T(32 keys x 16 queries)
// Every K or V fragment read from LDS feeds all RB row blocks. Each lane ends
// S^T holding the logits of ONE query (its column) for 4 keys of each tile.
// Taking the k index of the step as keys {4g..4g+3} of the first tile
// followed by {4g..4g+3} of the second (g = l/16) -- the sum over keys does
// not care about their order -- those logits' softmax weights are exactly
// the lane's own B operand for the V product, so no weight crosses lanes.
// V^T is read from LDS in that key order.
//
// Softmax: online, in base 2, with a lazily moved reference. A row's
// reference max m only moves when a step's max exceeds it by more than
// kMqSlack (log2 units), so the weights 2^(s - m) stay below 2^kMqSlack and
// the accumulators are rescaled only on such steps (and skipped by the whole
// wave when none of its rows moved). The result sum 2^(s-m) v / sum 2^(s-m)
// does not depend on m, so this is exact up to rounding. Steps whose keys lie
// below every row's limit in the wave skip the masking.
//
// Memory: each step's K and V tiles (32 keys x D, 2-byte) go from global
// memory straight into LDS (global_load_lds_dwordx4, no registers), read
// once per work-group, RD steps ahead of their use (kMqRing by default; the
// cascade's prefix work-groups take 1 to fit beside the decode items), into
// a ring of RD + 1 LDS buffers. Both tiles are row-major and swizzled so that
// their reads spread over the banks: in K the 16-byte chunk c of key row r
// sits at chunk c ^ (r % 16) (A-operand reads, 16 rows per pass), in V the
// 32-byte unit u at u ^ (r % 8) at head size 128 (transposed reads,
// ds_read_b64_tr_b16, which hand each lane one dimension of four keys, 8
// rows per pass). A wave's load fills 1 KB of a tile, each lane fetching the
// chunk that lands at its 16 bytes. A position with no slot loads a zero
// chunk. An FP8 (E4M3) cache goes through registers instead: each lane
// fetches its row's codes two steps ahead, converts them exactly to the
// query's 2-byte type and writes them into the same swizzled layout, so the
// products read the tiles the same way.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kMqWaves = 4;
constexpr int kMqRowsPerBlock = 16;           // query rows of one MFMA column block
constexpr int kMqStep = 32;                   // keys per MFMA step
constexpr float kMqEmptyMax = -1.0e30f;       // running max before any key (finite)
constexpr float kMqSlack = 8.f;               // lazy reference: weights stay <= 2^8
#ifndef PA_MQ_RING
#define PA_MQ_RING 2
#endif
constexpr int kMqRing = PA_MQ_RING;           // steps of K/V loads in flight
constexpr int kMqBufs = kMqRing + 1;          // LDS tiles: those, and the step computed

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <class DT> struct Mma;
template <> struct Mma<Fp16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  // Two weights in [0, 2^kMqSlack] rounded to nearest even, packed (lo, hi).
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};
template <> struct Mma<Bf16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// The four lanes that share a query column (lanes j, j+16, j+32, j+48), on
// the gfx950 lane swaps: v_permlane16_swap(x, x) leaves x of lanes l and
// l ^ 16 in its two results (in some order, per lane), v_permlane32_swap(x, x)
// those of l and l ^ 32. No LDS round trip.
__device__ __forceinline__ void mq_pair16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void mq_pair32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// max of two logits with v_max_f32 as is: the operands come out of the
// matrix core or the exp unit (never signalling NaNs), so the quieting that
// fmaxf adds around values from a lane swap is not needed.
__device__ __forceinline__ float mq_fmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float mq_max_over_groups(float x) {
  float a, b;
  mq_pair16(x, a, b);
  mq_pair32(mq_fmax(a, b), a, b);
  return mq_fmax(a, b);
}
__device__ __forceinline__ float mq_sum_over_groups(float x) {
  float a, b;
  mq_pair16(x, a, b);
  mq_pair32(a + b, a, b);
  return a + b;
}

// K and V tiles of NB steps (the ring of loads in flight plus the step
// computed), row-major (key, dimension), swizzled as described above.
template <int D, int NB = kMqBufs> struct MqLds {
  alignas(16) uint16_t k[NB][kMqStep][D];
  alignas(16) uint16_t v[NB][kMqStep][D];
};

// Source of the loads of positions that hold no key.
static __device__ __attribute__((aligned(16))) const uint32_t kMqZeroChunk[4] = {0u, 0u, 0u, 0u};

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at lds + 16 l, lds being the same for the whole wave.
// The compiler does not see this write: the reader waits with
// mq_wait_loads and a barrier.
__device__ __forceinline__ void mq_lds_load16(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}
// Until at most N of this wave's global loads are outstanding.
// The same with the non-temporal hint, for rows read once per launch.
__device__ __forceinline__ void mq_lds_load16_nt(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(lds) : "memory");
}
template <int N> __device__ __forceinline__ void mq_wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

typedef __attribute__((address_space(3))) char mq_lds_byte;
typedef __attribute__((address_space(3))) u32x4_t mq_lds_u32x4;
typedef short mq_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mq_i16x4 mq_lds_i16x4;
__device__ __forceinline__ mq_lds_byte* mq_lds_ptr(uint32_t a) {
  return reinterpret_cast<mq_lds_byte*>(a);
}
__device__ __forceinline__ u32x4_t mq_lds_read16(const mq_lds_byte* a) {
  return *reinterpret_cast<const mq_lds_u32x4*>(a);
}
// ds_read_b64_tr_b16: lane l of each 16-lane group receives, for y = 0..3,
// the 2-byte element at (address of group lane 4 y + (l % 16) / 4) +
// 2 * (l % 4): a 4 x 16 block of 2-byte elements read row-wise, transposed.
__device__ __forceinline__ uint2 mq_lds_read_tr16(const mq_lds_byte* a) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       reinterpret_cast<mq_lds_i16x4*>(const_cast<mq_lds_byte*>(a))));
}

// Running softmax state of one lane, per row block: its query column's
// reference max (identical in the column's four lanes), this lane's share of
// the exp-sum, and its C entries of O^T (dimensions 16*dt + 4*(lane/16) .. +3).
template <int D, int RB> struct MqState {
  f32x4_t acc[RB][D / 16];
  float m[RB], lsum[RB];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[b][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[b] = kMqEmptyMax;
      lsum[b] = 0.f;
    }
  }
};

template <bool B> struct MqFlag { static constexpr bool value = B; };

// Q^T as the B operand: this lane's query row q (D elements), k = 8*grp + 32*ks.
// With neg set every element's sign is flipped (exact in both 2-byte types):
// q.k * scale = (-q).k * |scale| for a negative scale, and the core takes
// scales >= 0 only. A row outside the batch (ok false) holds zeros. UNCOND:
// such a row reads the zero chunk instead of skipping its loads, so that no
// load is conditional and none is waited for before the loads the caller
// issues next.
template <int D, bool UNCOND = false>
__device__ __forceinline__ void mq_load_q(u32x4_t (&qb)[D / 32], const uint16_t* q, bool ok,
                                          bool neg) {
  const int grp = (threadIdx.x & 63) >> 4;
  const uint32_t flip = neg ? 0x80008000u : 0u;
  if constexpr (UNCOND) {
    const uint16_t* src = ok ? q + 8 * grp : reinterpret_cast<const uint16_t*>(kMqZeroChunk);
    const int step = ok ? 32 : 0;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qb[ks] = load_global16(src + step * ks) ^ flip;
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qb[ks] = ok ? *reinterpret_cast<const u32x4_t*>(q + 8 * grp + 32 * ks) : u32x4_t{0u, 0u, 0u, 0u};
      qb[ks] ^= flip;
    }
  }
}

// Attend every row of the work-group to positions [c0, kend) of kv head g.
// blk_of(t) gives the physical block of position t (c0 <= t < kend, asked
// with a wave-uniform t), or -1 for a skipped block, read as zeros;
// position t sits at slot blk * bs + t % bs. c0 is a multiple of 16 and of
// bs (>= 16), so the rows one wave's load slice covers (4 at head size 128,
// 8 at 64) never straddle a block.
// Keys >= row_end[b] are masked for this lane's row of block b; every
// position below kend must hold finite data (a position some row of the
// work-group may use). Must be reached by all threads of the work-group with
// the same c0 / kend (it synchronises); LDS is free again when it returns.
// sl2 (scale * log2 e) must be >= 0: mq_load_q folds a negative scale's sign
// into q. RD: steps of loads in flight (the ring holds RD + 1 steps). LEAN:
// read each V^T fragment just before its product instead of all of them
// before the softmax (32 fewer VGPRs at head size 128, for callers that
// share a register budget).
template <class DT, int D, int RB, int W = kMqWaves, int RD = kMqRing, bool LEAN = false,
          bool F8 = false, class BlkOf>
__device__ __forceinline__ void mq_attend(MqState<D, RB>& st, const u32x4_t (&qb)[RB][D / 32],
                                          MqLds<D, RD + 1>& lds, const void* kc, const void* vc,
                                          int64_t tok_stride, int g, int c0, int kend,
                                          const int (&row_end)[RB], float sl2, int bs,
                                          BlkOf blk_of) {
  constexpr int KS = D / 32;
  constexpr int DTILES = D / 16;
  constexpr int CH = D / 8;                    // 16-byte chunks of a row
  constexpr int CH16 = CH < 16 ? CH : 16;
  constexpr int TILE = kMqStep * D * 2;        // bytes of one K or V tile
  constexpr int SPW = TILE / 1024 / W;         // 1 KB tile slices each wave loads
  static_assert(SPW >= 1 && TILE % (1024 * W) == 0, "tile slices");
  constexpr int NB = RD + 1;
  static_assert(RD >= 1, "at least one step in flight");
  constexpr int DPS = 2 * SPW;                 // LDS loads a wave issues per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int grp = lane >> 4;
  const uint16_t* kbase = static_cast<const uint16_t*>(kc) + (int64_t)g * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(vc) + (int64_t)g * D;
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(kMqZeroChunk);
  const uint32_t stride32 = (uint32_t)tok_stride;   // Hkv * D < 2^31 elements

  // LDS byte addresses. Loads: slice u of this wave covers 16-byte units
  // 64 * (wave + W * u) + lane of a tile, i.e. key row dr[u], chunk dc[u].
  const uint32_t k0 = (uint32_t)(uintptr_t)&lds.k[0][0][0];
  const uint32_t v0 = (uint32_t)(uintptr_t)&lds.v[0][0][0];
  // The V tile swizzles 32-byte units (16 dimensions) instead: unit u of key
  // row r sits at u ^ vsw(r), so the 8 rows that half a wave's transposed
  // read touches fall on all 64 banks.
  constexpr int VU = D / 16;                   // 32-byte units per row
  constexpr int RPB = 128 / D;                 // rows per 256 bytes (one pass over the banks)
  auto vsw = [](int r) { return (r / RPB) % VU; };
  // Per slice: dr the lane's key row, lk / lv its element offset from the
  // slice's first row (row within the slice times the row stride, plus the
  // source chunk that lands at this lane's 16 bytes).
  int dr[SPW];
  uint32_t lk[SPW], lv[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int unit = 64 * (wave + W * u) + lane;
    const int cp = unit % CH;
    dr[u] = unit / CH;
    const uint32_t lrow = (uint32_t)(lane / CH) * stride32;
    lk[u] = lrow + (uint32_t)((cp ^ (dr[u] % CH16)) * 8);
    lv[u] = lrow + (uint32_t)((2 * ((cp >> 1) ^ vsw(dr[u])) + (cp & 1)) * 8);
  }
  // A operand of S^T: key row 16 kt + j, chunk grp + 4 ks (kt adds 16 rows).
  const mq_lds_byte* ka[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    ka[ks] = mq_lds_ptr(k0 + (j * D + ((grp + 4 * ks) ^ (j % CH16)) * 8) * 2);
  // A operand of O^T, transposed reads: group lane i = 4 y + q names key row
  // 4 grp + y (second read: + 16) and dimensions 16 dt + 4 q .. + 3, and this
  // lane receives dimension 16 dt + j of the four keys.
  const mq_lds_byte* va_addr[DTILES];
  {
    const int y = j >> 2, q = j & 3, r = 4 * grp + y;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
      va_addr[dt] = mq_lds_ptr(v0 + (r * D + (dt ^ vsw(r)) * 16 + q * 4) * 2);
  }

  // The wave's smallest row limit: a step entirely below it needs no mask;
  // its largest: a step entirely past it adds nothing to any of its rows.
  int wmin = row_end[0], wmax = row_end[0];
#pragma unroll
  for (int b = 1; b < RB; ++b) {
    wmin = min(wmin, row_end[b]);
    wmax = max(wmax, row_end[b]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    wmin = min(wmin, __shfl_xor(wmin, o));
    wmax = max(wmax, __shfl_xor(wmax, o));
  }
  wmin = __builtin_amdgcn_readfirstlane(wmin);
  wmax = __builtin_amdgcn_readfirstlane(wmax);

  // Step at t0 into LDS buffer buf; positions >= kend and skipped blocks
  // read the zero chunk (blk_of is only asked for positions in [c0, kend)).
  // A slice's block and the slot of its first row are wave-uniform.
  // The slices' block ids of the step at t0, read one step before its
  // loads are issued, so that the table read's latency hides behind a
  // step's products instead of delaying the issue.
  auto lookup = [&](int t0, int (&ids)[SPW]) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int tf = t0 + (64 * (wave + W * u)) / CH;      // the slice's first position
      ids[u] = tf < kend ? blk_of(tf) : -1;
    }
  };
  auto issue = [&](int t0, int buf, const int (&ids)[SPW]) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int tf = t0 + (64 * (wave + W * u)) / CH;      // the slice's first position
      const int blk = __builtin_amdgcn_readfirstlane(ids[u]);
      const bool ok = blk >= 0 && t0 + dr[u] < kend;
      const uint64_t base = (uint64_t)(uint32_t)(blk * bs + (tf & (bs - 1))) * stride32;
      const uint32_t dst = (uint32_t)(wave + W * u) * 1024 + (uint32_t)buf * TILE;
      mq_lds_load16(ok ? kbase + base + lk[u] : zero, k0 + dst);
      mq_lds_load16(ok ? vbase + base + lv[u] : zero, v0 + dst);
    }
  };
  auto compute = [&](int t0, int buf) {
    if (t0 >= wmax) return;                       // uniform: every key past the wave's rows
    const int bo = buf * TILE;
    f32x4_t c[RB][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int b = 0; b < RB; ++b) c[b][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t kv = mq_lds_read16(ka[ks] + bo + kt * 16 * D * 2);
#pragma unroll
        for (int b = 0; b < RB; ++b) c[b][kt] = Mma<DT>::run(kv, qb[b][ks], c[b][kt]);
      }
    }
    // V^T fragment of dimension tile dt: keys 4g .. 4g+3, then 16+4g .. 16+4g+3.
    auto read_va = [&](int dt) {
      const uint2 lo = mq_lds_read_tr16(va_addr[dt] + bo);
      const uint2 hi = mq_lds_read_tr16(va_addr[dt] + bo + 16 * D * 2);
      return u32x4_t{lo.x, lo.y, hi.x, hi.y};
    };
    // Unless LEAN, every fragment is read before the softmax, so the LDS
    // latency hides behind it.
    u32x4_t va[LEAN ? 1 : DTILES];
    if constexpr (!LEAN) {
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) va[dt] = read_va(dt);
    }
    u32x4_t pb[RB];
    float m_old[RB];
    bool moved = false;
    // One row block's weights. Unmasked, the scale is applied inside the
    // exponent's argument (one fma per key) and the max is taken on the raw
    // products: sl2 >= 0 and rounding is monotonic, so max(c) * sl2 is exactly
    // max(c * sl2).
    auto weights = [&](auto masked_tag) {
      constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        float lg[8];
        float mx;
        if constexpr (kMasked) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              lg[4 * kt + i] =
                  t0 + 16 * kt + 4 * grp + i < row_end[b] ? c[b][kt][i] * sl2 : -INFINITY;
          mx = lg[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) mx = fmaxf(mx, lg[i]);
        } else {
          mx = c[b][0][0];
#pragma unroll
          for (int i = 1; i < 8; ++i) mx = fmaxf(mx, c[b][i / 4][i % 4]);
          mx *= sl2;
        }
        // The reference moves only for a row with a key above it by more
        // than the slack. When no lane of the wave holds such a key (every
        // step after the first few), the row max across the lane groups is
        // not needed and the reference stays.
        m_old[b] = st.m[b];
        float mn = st.m[b];
        if (__ballot(mx > st.m[b] + kMqSlack) != 0) {   // uniform
          mx = mq_max_over_groups(mx);
          mn = mx > st.m[b] + kMqSlack ? mx : st.m[b];
        }
        moved |= mn != m_old[b];
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          p[i] = kMasked ? fast_exp2(lg[i] - mn) : fast_exp2(fmaf(c[b][i / 4][i % 4], sl2, -mn));
        st.m[b] = mn;
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[b][e] = Mma<DT>::pack(p[2 * e], p[2 * e + 1]);
      }
    };
    if (t0 + kMqStep <= wmin)                      // uniform: no key masked for any row
      weights(MqFlag<false>{});
    else
      weights(MqFlag<true>{});
    if (__ballot(moved) != 0) {                   // uniform: some row moved its reference
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const float alpha = fast_exp2(m_old[b] - st.m[b]);   // 1 where the row did not move
        st.lsum[b] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) st.acc[b][dt] *= alpha;
      }
    }
    // The exp-sum from the packed weights, as the product below sees them.
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) st.lsum[b] = Storage<DT>::dot2(pb[b][e], Storage<DT>::kOnes, st.lsum[b]);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const u32x4_t v = LEAN ? read_va(dt) : va[LEAN ? 0 : dt];
#pragma unroll
      for (int b = 0; b < RB; ++b) st.acc[b][dt] = Mma<DT>::run(v, pb[b], st.acc[b][dt]);
    }
  };

  // Step i lives in LDS buffer i % NB. Steps i + 1 .. i + RD - 1 are in
  // flight while step i computes; step i + RD goes into the buffer of step
  // i - 1, which every wave finished before the barrier of step i. With a
  // single step in flight it is issued right after that barrier, so that its
  // loads overlap step i's products; deeper rings issue it after them.
  // Steps past the range load zeros and are never computed, so the count of
  // loads in flight is the same at every step.
  const int nsteps = kend > c0 ? (kend - c0 + kMqStep - 1) / kMqStep : 0;
  if constexpr (F8) {
    // FP8 cache: lane rows fr of the step (the wave's RPW rows share a
    // block), EPT codes each from code fe on, fetched into registers two
    // steps ahead (register set step % 2) and converted into LDS buffer
    // step % 2 after the previous step's products. At the barrier of step i
    // every wave has written step i and finished reading step i - 1, whose
    // buffer then takes step i + 1.
    static_assert(RD == 1, "FP8 tiles: two LDS buffers");
    constexpr int EPT = kMqStep * D / (W * 64);   // codes per lane and tensor
    static_assert(EPT == 8 || EPT == 16, "FP8 staging layout");
    constexpr int LPRW = D / EPT;                 // lanes per key row
    constexpr int RPW = 64 / LPRW;                // key rows per wave
    typedef uint32_t f8row __attribute__((ext_vector_type(EPT / 4)));
    const int fr = wave * RPW + lane / LPRW;
    const int fe = (lane % LPRW) * EPT;
    const uint8_t* kb8 = static_cast<const uint8_t*>(kc) + (int64_t)g * D + fe;
    const uint8_t* vb8 = static_cast<const uint8_t*>(vc) + (int64_t)g * D + fe;
    const uint8_t* zero8 = reinterpret_cast<const uint8_t*>(kMqZeroChunk);
    // LDS byte addresses (buffer 0) of the lane's 16-byte chunks, swizzled as
    // the direct loads place them.
    uint32_t kdst[EPT / 8], vdst[EPT / 8];
#pragma unroll
    for (int cc = 0; cc < EPT / 8; ++cc) {
      const int sc = fe / 8 + cc;
      kdst[cc] = k0 + (uint32_t)(fr * D + (sc ^ (fr % CH16)) * 8) * 2;
      vdst[cc] = v0 + (uint32_t)(fr * D + (2 * ((sc >> 1) ^ vsw(fr)) + (sc & 1)) * 8) * 2;
    }
    auto fetch = [&](int t0, f8row& kr, f8row& vr) {
      const int tw = t0 + wave * RPW;              // the wave's first row
      const int blk = tw < kend ? __builtin_amdgcn_readfirstlane(blk_of(tw)) : -1;
      const bool ok = blk >= 0 && t0 + fr < kend;
      const uint64_t off = (uint64_t)(uint32_t)(blk * bs + ((t0 + fr) & (bs - 1))) * stride32;
      kr = *(const __attribute__((address_space(1))) f8row*)(ok ? kb8 + off : zero8);
      vr = *(const __attribute__((address_space(1))) f8row*)(ok ? vb8 + off : zero8);
    };
    auto land = [&](int buf, const f8row& kr, const f8row& vr) {
#pragma unroll
      for (int cc = 0; cc < EPT / 8; ++cc) {
        const u32x4_t kw = {Fp8Pair<DT>::template get<false>(kr[2 * cc]),
                            Fp8Pair<DT>::template get<true>(kr[2 * cc]),
                            Fp8Pair<DT>::template get<false>(kr[2 * cc + 1]),
                            Fp8Pair<DT>::template get<true>(kr[2 * cc + 1])};
        const u32x4_t vw = {Fp8Pair<DT>::template get<false>(vr[2 * cc]),
                            Fp8Pair<DT>::template get<true>(vr[2 * cc]),
                            Fp8Pair<DT>::template get<false>(vr[2 * cc + 1]),
                            Fp8Pair<DT>::template get<true>(vr[2 * cc + 1])};
        *reinterpret_cast<mq_lds_u32x4*>(mq_lds_ptr(kdst[cc] + (uint32_t)buf * TILE)) = kw;
        *reinterpret_cast<mq_lds_u32x4*>(mq_lds_ptr(vdst[cc] + (uint32_t)buf * TILE)) = vw;
      }
    };
    f8row kr8[2], vr8[2];
    if (nsteps > 0) fetch(c0, kr8[0], vr8[0]);
    if (nsteps > 1) fetch(c0 + kMqStep, kr8[1], vr8[1]);
    if (nsteps > 0) land(0, kr8[0], vr8[0]);
    if (nsteps > 2) fetch(c0 + 2 * kMqStep, kr8[0], vr8[0]);
    for (int i = 0; i < nsteps; i += 2) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int step = i + r;
        if (step >= nsteps) break;                // uniform
        __syncthreads();
        compute(c0 + step * kMqStep, r);
        if (step + 1 < nsteps) land(1 - r, kr8[1 - r], vr8[1 - r]);
        if (step + 3 < nsteps) fetch(c0 + (step + 3) * kMqStep, kr8[1 - r], vr8[1 - r]);
      }
    }
    __syncthreads();   // every read is done: LDS is free
    return;
  }
  constexpr bool kIssueFirst = RD == 1;
  int ids[SPW];
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    lookup(c0 + r * kMqStep, ids);
    issue(c0 + r * kMqStep, r, ids);
  }
  lookup(c0 + RD * kMqStep, ids);
  for (int i = 0; i < nsteps; i += NB) {
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int step = i + r;
      if (step >= nsteps) break;                  // uniform
      mq_wait_loads<(RD - 1) * DPS>();            // this wave's loads of this step
      __syncthreads();                            // everyone's
      if (kIssueFirst) {
        issue(c0 + (step + RD) * kMqStep, (r + RD) % NB, ids);
        lookup(c0 + (step + RD + 1) * kMqStep, ids);
      }
      compute(c0 + step * kMqStep, r);
      if (!kIssueFirst) {
        issue(c0 + (step + RD) * kMqStep, (r + RD) % NB, ids);
        lookup(c0 + (step + RD + 1) * kMqStep, ids);
      }
    }
  }
  mq_wait_loads<0>();
  __syncthreads();   // the last loads have landed and every read is done: LDS is free
}

}  // namespace pa
