// Cascade decode for a shared prefix, gfx950.
//
// When every sequence of the batch starts with the same physical blocks (a
// prompt prefix held once with a reference count per user: "01.
// PagedAttention 详解" §6, sharing through the block table), the decode step
// splits into
//   * the prefix part: the query rows of ALL sequences against the one copy
//     of the prefix's K/V. For each kv head this is a dense product of
//     (num_seqs * group) query rows with prefix_len keys, so it runs on the
//     matrix cores and reads the prefix from HBM once instead of once per
//     sequence;
//   * the suffix part: each sequence's own positions past the prefix, on the
//     ordinary partition kernel;
//   * the combine of both kinds of (max, exp-sum, weighted V) partials, with
//     the split-K algebra of the ordinary path.
// The result is the plain attention of every position < L (an exact
// reformulation, up to fp32 rounding and the 2-byte rounding of the
// softmax weights fed to the matrix cores).
//
// Prefix kernel layout. One work-group (4 waves) per (kv head, tile of 64
// query rows, chunk of 256 prefix keys); each wave owns 16 query rows. With
// v_mfma_f32_16x16x32 (lane l: A row l%16, B column l%16, k = 8*(l/16)..+7;
// C column l%16, rows 4*(l/16)..+3):
//   S^T(16 keys x 16 queries) = K(16 keys x D) . Q^T(D x 16 queries)
// leaves in each lane the logits of ONE query for 4 keys per 16-key tile.
// Those are exactly the softmax weights the same lane must supply as the B
// operand of
//   O^T(16 dims x 16 queries) += V^T(16 dims x 32 keys) . P^T(32 keys x 16 queries)
// when the k index of a 32-key step is taken as keys {4g..4g+3} of the first
// tile followed by {4g..4g+3} of the second (g = l/16); the sum over keys does
// not care about their order. V^T comes from LDS, where each step's V rows
// are stored transposed with that same key order readable as two 8-byte
// reads per lane. So no weight ever crosses lanes.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerWg = kWaves * kRowsPerWave;
constexpr int kStep = 32;                 // prefix keys per MFMA step
constexpr int kVRow = kStep / 2 + 6;      // LDS row (32-bit key pairs) of the transposed V
                                          // step; the padding keeps the staging writes and
                                          // the operand reads free of bank conflicts
constexpr float kEmptyMax = -1.0e30f;     // same sentinel as the partition kernel

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

__device__ __forceinline__ float wave_max_over_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <class DT, int D, int G>
__global__ __launch_bounds__(kWaves * 64) void cascade_prefix_kernel(const DecodeParams a) {
  using S = Storage<DT>;
  constexpr int NT = kWaves * 64;
  constexpr int KS = D / 32;            // MFMA k-steps over the head dimension
  constexpr int DTILES = D / 16;        // 16-dimension tiles of the output
  static_assert(D == 64 || D == 128, "head size");

  __shared__ int32_t s_tbl[kPrefixChunk / 16];
  __shared__ uint16_t s_k[2][kStep][D];
  __shared__ uint32_t s_v[2][D][kVRow];
  __shared__ int s_limit[kWaves];

  const int Hkv = a.num_kv_heads;
  int wg = blockIdx.x;
  const int g = wg % Hkv;
  wg /= Hkv;
  const int rt = wg % a.prefix_row_tiles;
  const int chunk = wg / a.prefix_row_tiles;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15;               // this lane's query column
  const int grp = lane >> 4;             // this lane's k group / C row group

  const int R = a.num_seqs * G;          // query rows of kv head g
  const int r = rt * kRowsPerWg + wave * kRowsPerWave + j;
  const bool row_ok = r < R;
  const int s = row_ok ? r / G : 0;
  const int h = g * G + (row_ok ? r % G : 0);

  const int c0 = chunk * kPrefixChunk;
  const int c1 = min(a.prefix_len, c0 + kPrefixChunk);
  int limit = 0;                          // keys this row may use: min(L, prefix_len)
  if (row_ok) {
    int L = a.lens[s];
    L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
    limit = min(L, a.prefix_len);
  }
  // The work-group's largest limit: V rows at or past it are not positions of
  // any of its sequences (possibly never written), so they are staged as 0.
  int wl = limit;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wl = max(wl, __shfl_xor(wl, o));
  if (lane == 0) s_limit[wave] = wl;

  const int lbs = a.log2_block_size;
  const int bs = a.block_size;
  const int b0 = c0 >> lbs;
  const int nb = (c1 - c0 + bs - 1) >> lbs;
  for (int i = tid; i < nb; i += NT) {    // row 0 of the tables holds the prefix
    const int blk = a.bt[b0 + i];
    s_tbl[i] = (uint64_t)(uint32_t)blk < (uint64_t)a.num_blocks ? blk : -1;  // corrupt: skip
  }
  __syncthreads();
  int wg_limit = s_limit[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) wg_limit = max(wg_limit, s_limit[w]);
  const int kend = min(c1, wg_limit);    // keys past this contribute nothing
  const int row_end = min(limit, c1);     // this row's keys in the chunk end here

  // Q^T as the B operand: column j = this row, k = 8*grp + 32*ks .. +7.
  u32x4_t qb[KS];
  {
    const uint16_t* qp = a.q + ((int64_t)s * a.num_q_heads + h) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks) : u32x4_t{0u, 0u, 0u, 0u};
  }

  const int64_t tok_stride = (int64_t)Hkv * D;
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc);
  const float sl2 = a.scale_log2;

  f32x4_t acc[DTILES];
#pragma unroll
  for (int t = 0; t < DTILES; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kEmptyMax, lsum = 0.f;

  // Physical slot of prefix position t (c0 <= t < c1); -1 for a skipped block.
  auto slot_of = [&](int t) -> int64_t {
    const int blk = s_tbl[(t >> lbs) - b0];
    return blk < 0 ? -1 : (int64_t)blk * bs + (t & (bs - 1));
  };

  // Each 32-key step's K and V rows are read from memory once per work-group
  // (coalesced 16-byte loads, two steps ahead of their use) and staged in a
  // double-buffered LDS area:
  //  - K row-major, the 16-byte chunk c of key row r at chunk c ^ (r % CH16):
  //    the A-operand reads (lane: key j, chunk grp + 4*ks) then spread over
  //    all banks;
  //  - V transposed, one 32-bit word per (dimension, key pair).
  constexpr int CH = D / 8;                    // 16-byte chunks of a row
  constexpr int CH16 = CH < 16 ? CH : 16;
  constexpr int KLOADS = kStep * CH / NT;      // K chunks per thread per step
  static_assert(KLOADS >= 1 && kStep * CH % NT == 0, "K staging");
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
      *reinterpret_cast<u32x4_t*>(&s_k[buf][r][(c ^ (r % CH16)) * 8]) = rg.k[u];
    }
    if (vthread) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_v[buf][vd + 2 * e][kp] = (rg.v[0][e] & 0xffffu) | (rg.v[1][e] << 16);
        s_v[buf][vd + 2 * e + 1][kp] = (rg.v[0][e] >> 16) | (rg.v[1][e] & 0xffff0000u);
      }
    }
  };
  auto compute = [&](int t0, int buf) {
    // S^T for the step's two 16-key tiles; lane: keys 16*kt + 4*grp + i, query j.
    float lg[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int r = 16 * kt + j;
      f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t kv =
            *reinterpret_cast<const u32x4_t*>(&s_k[buf][r][((grp + 4 * ks) ^ (r % CH16)) * 8]);
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
    mx = wave_max_over_groups(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * kt + i] = fast_exp2(lg[kt][i] - mn);
        ps += p[4 * kt + i];
      }
    lsum = fmaf(lsum, alpha, ps);
    m = mn;
    u32x4_t pb;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pb[e] = (uint32_t)S::from_float(p[2 * e]) | ((uint32_t)S::from_float(p[2 * e + 1]) << 16);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      acc[dt] *= alpha;
      const uint32_t* vr = &s_v[buf][16 * dt + j][2 * grp];
      const uint2 lo = *reinterpret_cast<const uint2*>(vr);       // keys 4g .. 4g+3
      const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);   // keys 16+4g .. 16+4g+3
      acc[dt] = Mma<DT>::run(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb, acc[dt]);
    }
  };

  // Steps i = 0, 1, ...: stage ring[i % 2] into LDS buffer i % 2, refill that
  // ring slot with step i + 2, then compute step i. One barrier per step: a
  // wave that stages step i has passed the barrier of step i - 1, which every
  // wave reaches only after computing step i - 2 from the same buffer.
  const int nsteps = kend > c0 ? (kend - c0 + kStep - 1) / kStep : 0;
  if (nsteps > 0) issue(c0, ring[0]);
  if (nsteps > 1) issue(c0 + kStep, ring[1]);
  for (int st = 0; st < nsteps; st += 2) {
    stage(ring[0], 0);
    if (st + 2 < nsteps) issue(c0 + (st + 2) * kStep, ring[0]);
    __syncthreads();
    compute(c0 + st * kStep, 0);
    if (st + 1 >= nsteps) break;
    stage(ring[1], 1);
    if (st + 3 < nsteps) issue(c0 + (st + 3) * kStep, ring[1]);
    __syncthreads();
    compute(c0 + (st + 1) * kStep, 1);
  }

  // Partial of this chunk for the row: (m, sum of weights, unnormalised O).
  lsum = wave_sum_over_groups(lsum);
  if (!row_ok) return;
  const int64_t pi = ((int64_t)s * a.num_q_heads + h) * a.part_stride + chunk;
  if (grp == 0) {
    a.ws_m[pi] = m;
    a.ws_l[pi] = lsum;
  }
  float* po = a.ws_o + pi * D + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt)
    *reinterpret_cast<float4*>(po + 16 * dt) =
        make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
}

template <class DT, int D, int G>
hipError_t launch_prefix(const DecodeParams& a, hipStream_t st) {
  const uint64_t nwg = (uint64_t)a.num_kv_heads * a.prefix_row_tiles * a.prefix_chunks;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffull) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((cascade_prefix_kernel<DT, D, G>), dim3((uint32_t)nwg), dim3(kWaves * 64), 0,
                     st, a);
  return hipGetLastError();
}

template <class DT, int D>
hipError_t launch_prefix_g(const DecodeParams& a, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_prefix<DT, D, 1>(a, st);
    case 2: return launch_prefix<DT, D, 2>(a, st);
    case 4: return launch_prefix<DT, D, 4>(a, st);
    case 8: return launch_prefix<DT, D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <class DT>
hipError_t launch_prefix_d(const DecodeParams& a, int head_size, int group, hipStream_t st) {
  switch (head_size) {
    case 64: return launch_prefix_g<DT, 64>(a, group, st);
    case 128: return launch_prefix_g<DT, 128>(a, group, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_cascade(const DecodeParams& a, int dtype, int head_size, int group,
                          hipStream_t stream) {
  const hipError_t e = dtype == 0 ? launch_prefix_d<Fp16>(a, head_size, group, stream)
                                  : launch_prefix_d<Bf16>(a, head_size, group, stream);
  if (e != hipSuccess) return e;
  return launch_decode(a, dtype, false, head_size, group, stream);
}

}  // namespace pa
