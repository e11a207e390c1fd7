// Multi-query paged attention core on the gfx950 matrix cores: many query rows
// that share a kv head, attended to a range of positions reached through a
// block table. Used by the cascade's shared-prefix kernel and by prefill.
//
// A work-group is 4 wave64s; each wave owns 16 query rows. With
// v_mfma_f32_16x16x32 (lane l: A row l%16, B column l%16, k = 8*(l/16)..+7;
// C column l%16, rows 4*(l/16)..+3) one 32-key step computes
//   S^T(16 keys x 16 queries)   = K(16 keys x D) . Q^T(D x 16 queries)   (two key tiles)
//   O^T(16 dims x 16 queries)  += V^T(16 dims x 32 keys) . P^T(32 keys x 16 queries)
// Each lane ends S^T holding the logits of ONE query (its column) for 4 keys
// of each tile. Taking the k index of the step as keys {4g..4g+3} of the first
// tile followed by {4g..4g+3} of the second (g = l/16) -- the sum over keys
// does not care about their order -- those logits' softmax weights are
// exactly the lane's own B operand for the V product, so no weight crosses
// lanes. V^T is read from LDS in that key order.
//
// Memory: each step's K and V rows are read once per work-group with
// coalesced 16-byte loads, two steps ahead of their use, into a
// double-buffered LDS area: K row-major with the 16-byte chunk c of key row r
// at chunk c ^ (r % 16) (the A-operand reads then spread over all banks), V
// transposed as one 32-bit word per (dimension, key pair) in padded rows.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kMqWaves = 4;
constexpr int kMqRowsPerWave = 16;
constexpr int kMqRowsPerWg = kMqWaves * kMqRowsPerWave;
constexpr int kMqStep = 32;                   // keys per MFMA step
constexpr int kMqVRow = kMqStep / 2 + 6;      // 32-bit key pairs per V^T row, padded
constexpr float kMqEmptyMax = -1.0e30f;       // running max before any key (finite)

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <class DT> struct Mma;
template <> struct Mma<Fp16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<Bf16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

// The four lanes that share a query column (lanes j, j+16, j+32, j+48).
__device__ __forceinline__ float mq_max_over_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float mq_sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int D> struct MqLds {
  uint16_t k[2][kMqStep][D];
  uint32_t v[2][D][kMqVRow];
};

// Running softmax state of one lane: its query column's max (identical in
// the column's four lanes), this lane's share of the exp-sum, and its C
// entries of O^T (dimensions 16*dt + 4*(lane/16) .. +3).
template <int D> struct MqState {
  f32x4_t acc[D / 16];
  float m, lsum;
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = kMqEmptyMax;
    lsum = 0.f;
  }
};

// Q^T as the B operand: this lane's query row q (D elements), k = 8*grp + 32*ks.
template <int D>
__device__ __forceinline__ void mq_load_q(u32x4_t (&qb)[D / 32], const uint16_t* q, bool ok) {
  const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qb[ks] = ok ? *reinterpret_cast<const u32x4_t*>(q + 8 * grp + 32 * ks) : u32x4_t{0u, 0u, 0u, 0u};
}

// Attend every row of the work-group to positions [c0, kend) of kv head g.
// slot_of(t) gives position t's physical slot (or -1: a skipped block, read
// as zeros). Keys >= row_end are masked for this lane's row; every position
// below kend must hold finite data (a position some row of the work-group
// may use). Must be reached by all threads of the work-group with the same
// c0 / kend (it synchronises); LDS is free again when it returns.
template <class DT, int D, class SlotOf>
__device__ __forceinline__ void mq_attend(MqState<D>& st, const u32x4_t (&qb)[D / 32],
                                          MqLds<D>& lds, const uint16_t* kc, const uint16_t* vc,
                                          int64_t tok_stride, int g, int c0, int kend, int row_end,
                                          float sl2, SlotOf slot_of) {
  using S = Storage<DT>;
  constexpr int NT = kMqWaves * 64;
  constexpr int KS = D / 32;
  constexpr int DTILES = D / 16;
  constexpr int CH = D / 8;                    // 16-byte chunks of a row
  constexpr int CH16 = CH < 16 ? CH : 16;
  constexpr int KLOADS = kMqStep * CH / NT;    // K chunks per thread per step
  static_assert(KLOADS >= 1 && kMqStep * CH % NT == 0, "K staging");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane & 15;
  const int grp = lane >> 4;
  const int kp = tid % 16;                     // V staging: key pair, 8 dimensions
  const int vd = (tid / 16) * 8;
  const bool vthread = tid < 16 * CH;
  struct Regs { u32x4_t k[KLOADS]; u32x4_t v[2]; };
  Regs ring[2];

  auto issue = [&](int t0, Regs& rg) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int idx = tid + NT * u;
      const int t = t0 + idx / CH;
      const int64_t sl = t < kend ? slot_of(t) : -1;
      rg.k[u] = sl >= 0 ? load_stream16(kc + sl * tok_stride + (int64_t)g * D + (idx % CH) * 8)
                        : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int t = t0 + 2 * kp + e;
      const int64_t sl = (vthread && t < kend) ? slot_of(t) : -1;
      rg.v[e] = sl >= 0 ? load_stream16(vc + sl * tok_stride + (int64_t)g * D + vd)
                        : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&](const Regs& rg, int buf) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int idx = tid + NT * u;
      const int r = idx / CH, c = idx % CH;
      *reinterpret_cast<u32x4_t*>(&lds.k[buf][r][(c ^ (r % CH16)) * 8]) = rg.k[u];
    }
    if (vthread) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lds.v[buf][vd + 2 * e][kp] = (rg.v[0][e] & 0xffffu) | (rg.v[1][e] << 16);
        lds.v[buf][vd + 2 * e + 1][kp] = (rg.v[0][e] >> 16) | (rg.v[1][e] & 0xffff0000u);
      }
    }
  };
  auto compute = [&](int t0, int buf) {
    float lg[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int r = 16 * kt + j;
      f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t kv =
            *reinterpret_cast<const u32x4_t*>(&lds.k[buf][r][((grp + 4 * ks) ^ (r % CH16)) * 8]);
        c = Mma<DT>::run(kv, qb[ks], c);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t0 + 16 * kt + 4 * grp + i;
        lg[kt][i] = key < row_end ? c[i] * sl2 : -INFINITY;
      }
    }
    float mx = lg[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, lg[kt][i]);
    mx = mq_max_over_groups(mx);
    const float mn = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - mn);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * kt + i] = fast_exp2(lg[kt][i] - mn);
        ps += p[4 * kt + i];
      }
    st.lsum = fmaf(st.lsum, alpha, ps);
    st.m = mn;
    u32x4_t pb;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pb[e] = (uint32_t)S::from_float(p[2 * e]) | ((uint32_t)S::from_float(p[2 * e + 1]) << 16);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      st.acc[dt] *= alpha;
      const uint32_t* vr = &lds.v[buf][16 * dt + j][2 * grp];
      const uint2 lo = *reinterpret_cast<const uint2*>(vr);       // keys 4g .. 4g+3
      const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);   // keys 16+4g .. 16+4g+3
      st.acc[dt] = Mma<DT>::run(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb, st.acc[dt]);
    }
  };

  // Steps i = 0, 1, ...: stage ring[i % 2] into LDS buffer i % 2, refill that
  // ring slot with step i + 2, then compute step i. One barrier per step: a
  // wave that stages step i has passed the barrier of step i - 1, which every
  // wave reaches only after computing step i - 2 from the same buffer.
  const int nsteps = kend > c0 ? (kend - c0 + kMqStep - 1) / kMqStep : 0;
  if (nsteps > 0) issue(c0, ring[0]);
  if (nsteps > 1) issue(c0 + kMqStep, ring[1]);
  for (int i = 0; i < nsteps; i += 2) {
    stage(ring[0], 0);
    if (i + 2 < nsteps) issue(c0 + (i + 2) * kMqStep, ring[0]);
    __syncthreads();
    compute(c0 + i * kMqStep, 0);
    if (i + 1 >= nsteps) break;
    stage(ring[1], 1);
    if (i + 3 < nsteps) issue(c0 + (i + 3) * kMqStep, ring[1]);
    __syncthreads();
    compute(c0 + (i + 1) * kMqStep, 1);
  }
  __syncthreads();   // the last step's LDS reads are done before LDS is reused
}

}  // namespace pa
