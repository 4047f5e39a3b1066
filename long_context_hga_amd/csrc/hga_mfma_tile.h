// Matrix-core pieces of the chunked-prefill attention, shared by the split
// kernel (one query chunk, partials merged afterwards) and the whole-prompt
// kernel (every query chunk of a prompt, online softmax over the tiles).
//
// A tile is 8 selected groups = 128 keys of one KV head, staged in LDS:
//   ks  [128 keys][D]  bf16 K rows, 16-byte chunk ch of key k at ch ^ (k % 16)
//   vt  [D][128 keys]  bf16 V^T rows; each 32-key quarter in the key order of
//                      the S^T entries (chunk qg holds keys 4qg + 0..3 and
//                      16 + 4qg + 0..3), chunk c of dim row r at c ^ (r % 16)
// A wave owns 16 query rows; lane (rl, qg) is C-layout column rl (its query
// row) and row group qg.  Contractions on v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T     A = 16 keys x 32 dims of K, B = the rotated query (bf16
//                   hi + lo, two products)
//   O^T += V^T P^T  A = 16 dims x 32 keys of V^T, B = the lane's own
//                   probabilities (hi + lo) in the key order S^T left them.
// FP8 pool (FP8 = true): the tile's E4M3FN codes are staged as bf16 (exact:
// every E4M3FN value is a bf16 value) and its 128 K and 128 V row scales go
// to LDS beside them; the K row scale multiplies the scores and the V row
// scale the probabilities (powers of two: exact), as in the decode kernel.
#pragma once

#include "hga_attend_common.h"

namespace hga {

constexpr int kTileGroups = kSplitGroups;                 // groups per tile
constexpr int kTileKeys = kTileGroups * kGroupTokens;     // 128 keys per tile

// 16 raw bytes of a tile row in flight (a vector type, so that arrays of them
// stay in registers across the loops that prefetch them)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The bf16 elements of x whose bit in keep (bit i = element i) is clear
// become +0.
__device__ __forceinline__ u32x4 keep_bf16x8(u32x4 x, uint32_t keep) {
  auto m = [&](int i) {
    return ((keep >> (2 * i)) & 1u ? 0x0000FFFFu : 0u) | ((keep >> (2 * i + 1)) & 1u ? 0xFFFF0000u : 0u);
  };
  return u32x4{x.x & m(0), x.y & m(1), x.z & m(2), x.w & m(3)};
}

// The lane's B operand of S^T = K Q^T is its query row at dims 32k + 8qg +
// 0..7 (k < 4): both halves of the RoPE pairs j = 8qg + i and 32 + 8qg + i
// (half-split pairs), or pairs 16k + 4qg + 0..3 whole (interleaved pairs),
// so the lane rotates its own operand.  qrow: the raw bf16 query row.
template <int D>
__device__ __forceinline__ void load_q_raw(const uint16_t* qrow, int qg, uint4 (&qraw)[D / 32]) {
#pragma unroll
  for (int k = 0; k < D / 32; ++k) qraw[k] = *reinterpret_cast<const uint4*>(qrow + 32 * k + 8 * qg);
}

// The RoPE frequencies of the lane's 16 query pairs, in the order rotate_q
// takes them: interleaved pairs, i = 4k + w is pair 16k + 4qg + w; half-split
// pairs, i = 8 half + 2w + e is pair 32 half + 8qg + 2w + e.  These are kernel
// arguments indexed by lane (vector loads): the caller issues them with the
// query loads so that the rotation, which runs while the K/V loads are in
// flight, does not wait for those.
template <int D>
__device__ __forceinline__ void load_q_omega(const KCfg& c, int qg, double (&om)[16]) {
  static_assert(D == 128, "16 RoPE pairs per lane");
#pragma unroll
  for (int i = 0; i < 16; ++i)
    om[i] = c.omega[c.interleaved ? 16 * (i >> 2) + 4 * qg + (i & 3) : 32 * (i >> 3) + 8 * qg + (i & 7)];
}

// Rotated, pre-scaled query of the lane's row at position tau: the angle
// tau * omega_j is formed in fp64 as a fraction of a turn and reduced exactly
// to [-1/2, 1/2]; sin and cos of the reduced turn run in fp32 (v_sin_f32 /
// v_cos_f32 take turns), within ~1e-6 rad.  The result is split into bf16
// hi + lo operands.
template <int D>
__device__ __forceinline__ void rotate_q(const KCfg& c, const uint4 (&qraw)[D / 32], const double (&om)[16],
                                         int tau, bf16x8 (&qop_hi)[D / 32], bf16x8 (&qop_lo)[D / 32]) {
  constexpr int KS = D / 32;
  const double tau_d = (double)tau;
  uint32_t hi[KS][4], lo[KS][4];
  if (c.interleaved) {
    // pairs (2j, 2j + 1): each 32-bit word of the operand holds one pair,
    // j = 16k + 4qg + w
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const uint32_t wv[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const double turns = tau_d * (om[4 * k + w] * 0.15915494309189533577);
        const float fr = (float)(turns - rint(turns));
        const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
        const float x = __uint_as_float(wv[w] << 16);
        const float y = __uint_as_float(wv[w] & 0xFFFF0000u);
        split_pair((x * cs - y * sn) * c.qscale_log2, (x * sn + y * cs) * c.qscale_log2, hi[k][w], lo[k][w]);
      }
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qop_hi[k] = __builtin_bit_cast(bf16x8, make_uint4(hi[k][0], hi[k][1], hi[k][2], hi[k][3]));
      qop_lo[k] = __builtin_bit_cast(bf16x8, make_uint4(lo[k][0], lo[k][1], lo[k][2], lo[k][3]));
    }
    return;
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {  // pairs j = 32*half + 8qg + i
    const uint32_t wx[4] = {qraw[half].x, qraw[half].y, qraw[half].z, qraw[half].w};
    const uint32_t wy[4] = {qraw[half + 2].x, qraw[half + 2].y, qraw[half + 2].z, qraw[half + 2].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // pairs i = 2w, 2w + 1: one packed register each
      float rx[2], ry[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const double turns = tau_d * (om[8 * half + 2 * w + e] * 0.15915494309189533577);
        const float fr = (float)(turns - rint(turns));
        const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
        const float x = __uint_as_float(e ? (wx[w] & 0xFFFF0000u) : (wx[w] << 16));
        const float y = __uint_as_float(e ? (wy[w] & 0xFFFF0000u) : (wy[w] << 16));
        rx[e] = (x * cs - y * sn) * c.qscale_log2;
        ry[e] = (x * sn + y * cs) * c.qscale_log2;
      }
      split_pair(rx[0], rx[1], hi[half][w], lo[half][w]);
      split_pair(ry[0], ry[1], hi[half + 2][w], lo[half + 2][w]);
    }
  }
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    qop_hi[k] = __builtin_bit_cast(bf16x8, make_uint4(hi[k][0], hi[k][1], hi[k][2], hi[k][3]));
    qop_lo[k] = __builtin_bit_cast(bf16x8, make_uint4(lo[k][0], lo[k][1], lo[k][2], lo[k][3]));
  }
}

// Threads that stage a tile: NTHR = 256 (one workgroup of 4 waves) or 512.
// Thread tid stages groups it = i * (NTHR / 256) + tid / 256 (i < GPT) with
// the 256-thread maps below applied to sub = tid % 256.
template <int NTHR>
struct TileStaging {
  static_assert(NTHR == 256 || NTHR == 512, "tile staging threads");
  static constexpr int R = NTHR / 256;               // threads per 256-thread map slot
  static constexpr int GPT = kTileGroups / R;        // groups per thread
  template <class X>
  __device__ static __forceinline__ X pick(const X (&a)[kTileGroups], int i, int half) {
    if constexpr (R == 1) return a[i];
    else return half ? a[R * i + 1] : a[R * i];
  }
};

// Global loads of a tile (all groups issued together; a missing group's
// base is any in-range row, masked later):
//   K: group it, sub = (row sub/16, 16-byte chunk sub%16)
//   V: group it's V^T block ([D][16], as the pool stores it), sub = (dim
//      sub/2, tokens 8*(sub%2) .. +7)
// FP8: the same elements as codes (8 bytes per load, in .x and .y), and the
// row scale of key tid (tid < 128: K) or key tid - 128 (tid < 256: V) of the
// tile in sc; scales of the pool rows follow its codes (k_sc, v_sc).
template <int D, int NTHR = 256, bool FP8 = false>
__device__ __forceinline__ void load_tile(const void* k, const void* v,
                                          const size_t (&gbase)[kTileGroups], int tid,
                                          u32x4 (&kraw)[TileStaging<NTHR>::GPT],
                                          u32x4 (&vraw)[TileStaging<NTHR>::GPT],
                                          const float* k_sc = nullptr, const float* v_sc = nullptr,
                                          float* sc = nullptr) {
  using TS = TileStaging<NTHR>;
  constexpr int CH = D / 8;
  const int sub = tid % 256, half = tid / 256;
  if constexpr (FP8) {
    const uint8_t* kc = static_cast<const uint8_t*>(k);
    const uint8_t* vc = static_cast<const uint8_t*>(v);
#pragma unroll
    for (int i = 0; i < TS::GPT; ++i) {
      const uint2 x = *reinterpret_cast<const uint2*>(kc + TS::pick(gbase, i, half) + (size_t)(sub / CH) * D + (sub % CH) * 8);
      kraw[i] = u32x4{x.x, x.y, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < TS::GPT; ++i) {
      const uint2 x = *reinterpret_cast<const uint2*>(vc + TS::pick(gbase, i, half) + (size_t)(sub >> 1) * kGroupTokens + 8 * (sub & 1));
      vraw[i] = u32x4{x.x, x.y, 0u, 0u};
    }
    if (tid < 2 * kTileKeys) {  // key = tid % 128 of the tile: group key / 16, token key % 16
      const int key = tid % kTileKeys;
      const size_t row = gbase[key / kGroupTokens] / D + key % kGroupTokens;
      *sc = tid < kTileKeys ? k_sc[row] : v_sc[row];
    }
  } else {
    const uint16_t* kb = static_cast<const uint16_t*>(k);
    const uint16_t* vb = static_cast<const uint16_t*>(v);
#pragma unroll
    for (int i = 0; i < TS::GPT; ++i)
      kraw[i] = *reinterpret_cast<const u32x4*>(kb + TS::pick(gbase, i, half) + (size_t)(sub / CH) * D + (sub % CH) * 8);
#pragma unroll
    for (int i = 0; i < TS::GPT; ++i)
      vraw[i] = *reinterpret_cast<const u32x4*>(vb + TS::pick(gbase, i, half) + (size_t)(sub >> 1) * kGroupTokens + 8 * (sub & 1));
  }
}

// 8 E4M3FN codes (x.x, x.y) -> the same 8 values as bf16 (exact)
__device__ __forceinline__ u32x4 fp8x8_bf16(u32x4 x) {
  const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.x, false);
  const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.x, true);
  const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.y, false);
  const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.y, true);
  return u32x4{pack_bf16x2(f0[0], f0[1]), pack_bf16x2(f1[0], f1[1]), pack_bf16x2(f2[0], f2[1]),
               pack_bf16x2(f3[0], f3[1])};
}

// The loaded tile into LDS.  V of a key that is missing (gpos < 0) or lies
// after pos_last is stored as zero: an unwritten pool row may hold NaN, and
// 0 x NaN would poison the product.  all_before (uniform): every group is
// present and ends before the first query position, so nothing is masked.
// FP8: codes become bf16 here, and the row scales (sc from load_tile) go to
// sc_k / sc_v [128] (the V scale of a key that is masked as above is stored
// as zero, so that it meets its zero probability as a zero).
template <int D, int NTHR = 256, bool FP8 = false>
__device__ __forceinline__ void stage_tile(uint16_t* ks, uint16_t* vt,
                                           const u32x4 (&kraw)[TileStaging<NTHR>::GPT],
                                           const u32x4 (&vraw)[TileStaging<NTHR>::GPT],
                                           const int (&gpos)[kTileGroups], int pos_last, int tid,
                                           bool all_before, float sc = 0.f, float* sc_k = nullptr,
                                           float* sc_v = nullptr) {
  using TS = TileStaging<NTHR>;
  constexpr int CH = D / 8;
  const int sub = tid % 256, half = tid / 256;
  if constexpr (FP8) {
    if (tid < kTileKeys) {
      sc_k[tid] = sc;
    } else if (tid < 2 * kTileKeys) {
      const int key = tid - kTileKeys, gp = gpos[key / kGroupTokens];
      const bool keep = all_before || (gp >= 0 && gp + key % kGroupTokens <= pos_last);
      sc_v[key] = keep ? sc : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < TS::GPT; ++i) {
    const int it = TS::R * i + half;
    const int key = it * kGroupTokens + sub / CH, ch = sub % CH;
    *reinterpret_cast<u32x4*>(ks + key * D + (ch ^ (key % CH)) * 8) = FP8 ? fp8x8_bf16(kraw[i]) : kraw[i];
  }
  const int dim = sub >> 1, hf = sub & 1;
#pragma unroll
  for (int i = 0; i < TS::GPT; ++i) {
    const int it = TS::R * i + half;
    u32x4 x = FP8 ? fp8x8_bf16(vraw[i]) : vraw[i];
    if (!all_before) {  // uniform
      const int gp = TS::pick(gpos, i, half);
      uint32_t keep = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) keep |= (gp >= 0 && gp + 8 * hf + e <= pos_last) ? (1u << e) : 0u;
      x = keep_bf16x8(x, keep);
    }
    // keys 16*(it%2) + 8hf + 0..7 of quarter it/2: column groups 2hf and
    // 2hf + 1, half it%2 of their chunks
    const int c0 = 4 * (it >> 1) + 2 * hf, h = 4 * (it & 1);
    *reinterpret_cast<uint2*>(vt + dim * kTileKeys + ((c0 ^ (dim & 15)) * 8) + h) = make_uint2(x.x, x.y);
    *reinterpret_cast<uint2*>(vt + dim * kTileKeys + (((c0 + 1) ^ (dim & 15)) * 8) + h) = make_uint2(x.z, x.w);
  }
}

// S^T of the staged tile for the wave's rows: s[t][n][i] = score (log2
// units) of key 32t + 16n + 4qg + i for the lane's query row at position
// tau, -inf where the key is not visible (missing group, or after tau; with
// all_before every key is visible).
// Returns the lane's maximum; the row maximum needs rows_max.  The operand
// reads of quarter t + 1 are issued before the products of quarter t
// (scheduling barriers keep that order), so LDS latency hides under the
// matrix-core work.
template <int D, bool FP8 = false>
__device__ __forceinline__ float tile_scores(const uint16_t* ks, const bf16x8 (&qop_hi)[D / 32],
                                             const bf16x8 (&qop_lo)[D / 32],
                                             const int (&gpos)[kTileGroups], int tau, int rl, int qg,
                                             f32x4 (&s)[4][2], bool all_before,
                                             const float* sc_k = nullptr) {
  constexpr int KS = D / 32;
  constexpr int NT = kTileGroups / 2;
  auto load_k = [&](int t, bf16x8 (&kop)[2][KS]) {
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int k = 0; k < KS; ++k)
        kop[n][k] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(ks + (32 * t + 16 * n + rl) * D + (((4 * k + qg) ^ rl) * 8)));
  };
  bf16x8 kop[2][2][KS];
  load_k(0, kop[0]);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t + 1 < NT) load_k(t + 1, kop[(t + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    s[t][0] = s[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
        s[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[t & 1][n][k], qop_hi[k], s[t][n], 0, 0, 0);
#pragma unroll
      for (int n = 0; n < 2; ++n)
        s[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[t & 1][n][k], qop_lo[k], s[t][n], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (FP8) {  // the K row scale of key 32t + 16n + 4qg + i
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const float4 kq = *reinterpret_cast<const float4*>(sc_k + 32 * t + 16 * n + 4 * qg);
        s[t][n][0] *= kq.x;
        s[t][n][1] *= kq.y;
        s[t][n][2] *= kq.z;
        s[t][n][3] *= kq.w;
      }
  }
  float tmax = -INFINITY;
  if (!all_before) {  // uniform
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int gp = gpos[2 * t + n];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = gp >= 0 && gp + 4 * qg + i <= tau;
          s[t][n][i] = vis ? s[t][n][i] : -INFINITY;
        }
      }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[t][n][i]);
  return tmax;
}

// Probabilities p = 2^(s - mref) of the tile (added to the lane's l) and
// O^T += V^T P^T.  The V^T operand reads of quarter t + 1 are issued with
// the products of quarter t.
template <int D, bool FP8 = false>
__device__ __forceinline__ void tile_pv(const uint16_t* vt, const f32x4 (&s)[4][2], float mref, int rl,
                                        int qg, float& l, f32x4 (&o)[D / 16],
                                        const float* sc_v = nullptr) {
  constexpr int NB = D / 16;
  constexpr int NT = kTileGroups / 2;
  auto load_v = [&](int t, bf16x8 (&vop)[NB]) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      vop[n] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(vt + (16 * n + rl) * kTileKeys + (((4 * t + qg) ^ rl) * 8)));
  };
  // k-slot 4n + i of quarter t is key 32t + 16n + 4qg + i
  auto probs = [&](int t, bf16x8& hi, bf16x8& lo) {
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float p0 = __builtin_amdgcn_exp2f(s[t][k >> 1][2 * (k & 1)] - mref);
      float p1 = __builtin_amdgcn_exp2f(s[t][k >> 1][2 * (k & 1) + 1] - mref);
      l += p0 + p1;
      if constexpr (FP8) {  // the V row scale joins the probability
        const int key = 32 * t + 16 * (k >> 1) + 4 * qg + 2 * (k & 1);
        p0 *= sc_v[key];
        p1 *= sc_v[key + 1];
      }
      split_pair(p0, p1, ph[k], pl[k]);
    }
    hi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
  };
  // The probabilities of quarter t + 1 are computed while the products of
  // quarter t run on the matrix core (one product, then a few vector
  // instructions, in turn).
  bf16x8 vop[2][NB];
  bf16x8 pop_hi[2], pop_lo[2];
  load_v(0, vop[0]);
  probs(0, pop_hi[0], pop_lo[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int cur = t & 1, nxt = cur ^ 1;
    if (t + 1 < NT) {
      load_v(t + 1, vop[nxt]);
      probs(t + 1, pop_hi[nxt], pop_lo[nxt]);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n)
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[cur][n], pop_hi[cur], o[n], 0, 0, 0);
#pragma unroll
    for (int n = 0; n < NB; ++n)
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[cur][n], pop_lo[cur], o[n], 0, 0, 0);
    if (t + 1 < NT) {
#pragma unroll
      for (int i = 0; i < 2 * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix product
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three vector ALU instructions
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace hga
