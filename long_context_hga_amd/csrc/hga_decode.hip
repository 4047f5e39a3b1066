// Exact softmax attention over the selected token K/V, decode shape (1..15
// query tokens), on the matrix cores.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4: after
// routing, the output is softmax attention over the exact token K/V of the
// selected set; no summary value enters it.
//
// Why matrix cores for decode: with grouped-query attention every K/V byte
// meets Hg query heads.  At Hg = 8 a 512-byte token row (K + V, d = 128) costs
// 2 * 128 * 8 = 2048 FMAs, 4 FMA per byte: the VALU (39 T lane-ops/s
// unpacked) would need longer than HBM (8 TB/s) takes to deliver the bytes,
// so the contraction itself, [Hg query rows x d] against [d x keys], goes to
// v_mfma_f32_16x16x32_bf16 and the kernel stays bound by the loads.
//
// Work split: grid = (splits of 8 selected groups, Hkv, B * column blocks),
// 256 threads.  A column block is 16 query rows (query head, query token) of
// one KV head; wave w owns 2 groups (32 keys) of the split.  Every K/V load
// of a wave is issued before anything else, straight from the pool into the
// registers that feed the matrix cores:
//   S^T = K Q^T   A = K rows (16 B per lane per k-step, row-major pool).  The
//                 16 rows of block n are the keys 8*(r/4) + 4n + r%4, so that
//                 the C layout leaves each lane 8 consecutive keys of its
//                 query row: keys 8q..8q+7 for lane group q.
//   O^T = V^T P^T A = V^T (the pool stores each 16-token group transposed, so
//                 the 8 consecutive keys of a dim are 16 contiguous bytes),
//                 B = the lane's own probabilities, unmoved.
// The query is rotated once per workgroup (fp64 angle reduced to a fraction
// of a turn, hardware sin/cos, ~1e-6 rad), scaled by log2(e)/sqrt(d) and
// split into bf16 hi + lo operands (two products, ~2^-17 relative).  An fp32
// pool is split the same way (three products).  The four waves' (max, sum,
// output) merge through LDS into one partial (m, l, o) per query row and
// split; the merge kernel combines the splits exactly.  Keys after a query
// token are masked, and V of a key that is missing or not yet written is
// zeroed before it meets a zero probability.
#include "hga_attend_common.h"
#include "hga_gather_dev.h"

namespace hga {

constexpr int kColRows = 16;  // query rows per column block

// 16 bytes of K or V read once per step: a non-temporal load (the rows are
// not reused, so they need not displace cached lines)
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load_stream8(const void* p) {  // 8 bytes read once
  const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
  return make_uint2(v.x, v.y);
}

// 8 fp32 values (two uint4) -> bf16x8 hi and lo operands
__device__ __forceinline__ void split8(const uint4& x0, const uint4& x1, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
  split_pair(__uint_as_float(x0.x), __uint_as_float(x0.y), h[0], l[0]);
  split_pair(__uint_as_float(x0.z), __uint_as_float(x0.w), h[1], l[1]);
  split_pair(__uint_as_float(x1.x), __uint_as_float(x1.y), h[2], l[2]);
  split_pair(__uint_as_float(x1.z), __uint_as_float(x1.w), h[3], l[3]);
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct DecodeShared {
  uint16_t qhi[kColRows][D + 8];  // rotated, scaled query rows, bf16 hi part
  uint16_t qlo[kColRows][D + 8];  // and lo part
  float mw[4][kColRows];          // per-wave row maxima
  float lw[4][kColRows];          // per-wave row sums (rescaled)
  float ob[4][kColRows][D + 4];   // per-wave output rows (rescaled)
};

// 8 E4M3FN codes -> the same 8 values as bf16 (exact: every E4M3FN value is a
// bf16 value), via v_cvt_pk_f32_fp8.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 c) {
  const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false);
  const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
  const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false);
  const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
  return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(f0[0], f0[1]), pack_bf16x2(f1[0], f1[1]),
                                               pack_bf16x2(f2[0], f2[1]), pack_bf16x2(f3[0], f3[1])));
}

// One split workgroup (256 threads): split `split` of KV head h, grid row bz
// = sequence * column blocks + column block.  FP8: the pool holds E4M3FN
// codes with power-of-two row scales (bf16 inputs): the codes enter the
// matrix cores as bf16, the K row scale multiplies the scores and the V row
// scale the probabilities (both exact).
template <int D, int HG, bool BF16, bool FP8 = false>
__device__ __forceinline__ void decode_split(const AttendArgs& args, int split, int h, int bz) {
  constexpr int P = D / 2;
  constexpr int KS = D / 32;          // k-steps of QK^T
  constexpr int NB = D / 16;          // 16-dim blocks of the output
  constexpr int NRG = 256 / P;        // row groups of the rotation
  constexpr int RPT = kColRows / NRG; // rows rotated per thread
  constexpr int EV = BF16 ? 1 : 2;    // uint4 per 8 elements
  __shared__ __align__(16) DecodeShared<D> sh;

  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  // every kernel argument used below, read from the argument segment at once
  // (one scalar round trip, instead of one at each first use)
  asm volatile("" ::"s"(c.lists), "s"(c.kvdiv), "s"(c.hq), "s"(c.hkv), "s"(c.n_sink),
               "s"(c.n_local), "s"(c.interleaved), "s"(c.qscale_log2), "s"(a.lq), "s"(a.max_sel),
               "s"(a.src_layout), "s"(a.src_cap), "s"(a.part_sel), "s"(a.two_part),
               "s"(args.n_splits), "s"(a.B), "s"(a.q), "s"(a.q_pos0), "s"(a.k), "s"(a.v),
               "s"(a.sel), "s"(a.n_sel), "s"(a.part));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane & 15, qg = lane >> 4;
  const int n_rows = HG * a.lq;
  const int ncb = (n_rows + kColRows - 1) / kColRows;
  const int b = bz / ncb, cb = bz % ncb;
  const int unit = b * c.lists + h;               // the list (and its partial records)
  const int unit_p = b * c.hkv + h / c.kvdiv;       // the pool rows of its KV head
  const int pos0 = a.q_pos0[b];
  const int n_sel = a.n_sel[unit];
  const int* sel = a.sel + (size_t)unit * a.max_sel;
  const int v0 = split * kSplitGroups + 2 * wave;  // this wave's first list position
  int sel_spec[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) sel_spec[g] = sel[v0 + g < a.max_sel ? v0 + g : a.max_sel - 1];
  // raw query pairs (j, j+P) of the rows this thread rotates
  const int jr = tid % P, rg = tid / P;
  uint32_t qx[RPT], qy[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    int gr = cb * kColRows + rg + NRG * i;
    gr = gr < n_rows ? gr : n_rows - 1;
    const int tq = gr / HG, hh = gr % HG;
    const size_t row = ((size_t)(b * c.hq + h * HG + hh) * a.lq + tq) * D;
    if constexpr (BF16) {
      qx[i] = static_cast<const uint16_t*>(a.q)[row + pair_a(c, jr)];
      qy[i] = static_cast<const uint16_t*>(a.q)[row + pair_b(c, jr)];
    } else {
      qx[i] = __float_as_uint(static_cast<const float*>(a.q)[row + pair_a(c, jr)]);
      qy[i] = __float_as_uint(static_cast<const float*>(a.q)[row + pair_b(c, jr)]);
    }
  }
  // the RoPE frequency of pair jr (a kernel argument indexed by lane, so a
  // vector load): issued with the query loads, ahead of the K/V loads, so
  // that the rotation below does not wait for them
  const double nu = c.omega[jr] * 0.15915494309189533577;  // turns per position

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    bad = lp.n_routed < 0;
  }
  if (bad) return;  // the merge kernel writes NaN for this unit
  const int n_part = part_count(a.part_sel, lp, n_sel);
  if (split * kSplitGroups >= n_part) return;  // an empty split: the merge kernel skips it
  const int pos_last = pos0 + a.lq - 1;

  // ---- this wave's two groups: first position (-1: none) and source rows
  int gpos[2];
  size_t kb[2], vb[2];
  {
    const int max_gid = a.src_cap / kGroupTokens - 1;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int v = v0 + g;
      const int slot = part_slot(a.part_sel, lp, v < n_part ? v : split * kSplitGroups);
      int gid = a.part_sel == HGA_PART_ALL ? sel_spec[g] : sel[slot];
      const bool in_range = gid >= 0 && (a.src_layout == HGA_SRC_WORKING_SET || gid <= max_gid);
      gpos[g] = (v < n_part && in_range) ? gid * kGroupTokens : -1;
      gid = gid < 0 ? 0 : (gid > max_gid ? max_gid : gid);
      const size_t blk = a.src_layout == HGA_SRC_WORKING_SET
                             ? ((size_t)unit * a.max_sel + slot)
                             : ((size_t)unit_p * (a.src_cap / kGroupTokens) + gid);
      kb[g] = blk * kGroupTokens * D;  // K rows of the group, row-major
      vb[g] = blk * kGroupTokens * D;  // V^T block of the group, [D][16]
    }
  }
  // ---- every K/V load of the wave
  //   K (A of S^T): block n, lane row rl -> key 8*(rl/4) + 4n + rl%4 of the
  //   wave's 32, i.e. group rl/8, token 8*((rl/4)%2) + 4n + rl%4
  //   V^T (A of O^T): dim 16*blk + rl, keys 8qg..8qg+7 = group qg/2,
  //   tokens 8*(qg%2)..+7
  uint4 kraw[2][KS][EV], vraw[NB][EV];
  uint2 k8[2][KS], v8[NB];  // FP8: 8 codes per operand
  float ksc[8], vsc[8];     // FP8: row scales of the lane's keys 8qg .. 8qg + 7
  if constexpr (FP8) {
    const uint8_t* kc = static_cast<const uint8_t*>(a.k);
    const uint8_t* vc = static_cast<const uint8_t*>(a.v);
    const size_t kbase = (rl >> 3) ? kb[1] : kb[0];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int t = 8 * ((rl >> 2) & 1) + 4 * n + (rl & 3);
#pragma unroll
      for (int k = 0; k < KS; ++k)
        k8[n][k] = load_stream8(kc + kbase + (size_t)t * D + 32 * k + 8 * qg);
    }
    const size_t vbase = (qg >> 1) ? vb[1] : vb[0];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      v8[nb] = load_stream8(vc + vbase + (size_t)(16 * nb + rl) * kGroupTokens + 8 * (qg & 1));
    // the scales follow the codes of every pool (or working-set) unit; row =
    // group row * 16 + token
    const size_t codes =
        (size_t)a.B * (a.src_layout == HGA_SRC_WORKING_SET ? c.lists : c.hkv) * a.src_cap * D;
    const size_t srow = ((qg >> 1) ? kb[1] : kb[0]) / D + 8 * (qg & 1);
    const float4* kq = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(kc + codes) + srow);
    const float4* vq = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(vc + codes) + srow);
    const float4 k0 = kq[0], k1 = kq[1], w0 = vq[0], w1 = vq[1];
    ksc[0] = k0.x; ksc[1] = k0.y; ksc[2] = k0.z; ksc[3] = k0.w;
    ksc[4] = k1.x; ksc[5] = k1.y; ksc[6] = k1.z; ksc[7] = k1.w;
    vsc[0] = w0.x; vsc[1] = w0.y; vsc[2] = w0.z; vsc[3] = w0.w;
    vsc[4] = w1.x; vsc[5] = w1.y; vsc[6] = w1.z; vsc[7] = w1.w;
  } else {
    const int gk = rl >> 3;
    const size_t kbase = gk ? kb[1] : kb[0];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int t = 8 * ((rl >> 2) & 1) + 4 * n + (rl & 3);
#pragma unroll
      for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          const size_t off = kbase + (size_t)t * D + 32 * k + 8 * qg + 4 * e;
          kraw[n][k][e] = BF16 ? load_stream(static_cast<const uint16_t*>(a.k) + off)
                               : load_stream(static_cast<const float*>(a.k) + off);
        }
    }
    const size_t vbase = (qg >> 1) ? vb[1] : vb[0];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        const size_t off = vbase + (size_t)(16 * nb + rl) * kGroupTokens + 8 * (qg & 1) + 4 * e;
        vraw[nb][e] = BF16 ? load_stream(static_cast<const uint16_t*>(a.v) + off)
                           : load_stream(static_cast<const float*>(a.v) + off);
      }
  }

  // ---- rotated, pre-scaled query rows of this column block -> LDS (bf16
  // hi, lo); rows past the last (head, token) are zero
  {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + NRG * i;
      const int gr = cb * kColRows + r;
      float rx = 0.f, ry = 0.f;
      if (gr < n_rows) {
        const double turns = (double)(pos0 + gr / HG) * nu;
        const float fr = (float)(turns - rint(turns));
        const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
        const float x = BF16 ? __uint_as_float(qx[i] << 16) : __uint_as_float(qx[i]);
        const float y = BF16 ? __uint_as_float(qy[i] << 16) : __uint_as_float(qy[i]);
        rx = (x * cs - y * sn) * c.qscale_log2;
        ry = (x * sn + y * cs) * c.qscale_log2;
      }
      uint32_t hi, lo;
      split_pair(rx, ry, hi, lo);
      sh.qhi[r][pair_a(c, jr)] = (uint16_t)(hi & 0xFFFFu);
      sh.qhi[r][pair_b(c, jr)] = (uint16_t)(hi >> 16);
      sh.qlo[r][pair_a(c, jr)] = (uint16_t)(lo & 0xFFFFu);
      sh.qlo[r][pair_b(c, jr)] = (uint16_t)(lo >> 16);
    }
  }
  __syncthreads();
  bf16x8 qop_hi[KS], qop_lo[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    qop_hi[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sh.qhi[rl][32 * k + 8 * qg]));
    qop_lo[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sh.qlo[rl][32 * k + 8 * qg]));
  }
  const int grow = cb * kColRows + rl;                       // this lane's query row
  const int tau = pos0 + (grow < n_rows ? grow / HG : a.lq - 1);

  float m = -INFINITY, l = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (gpos[0] >= 0 || gpos[1] >= 0) {  // wave-uniform
    // ---- S^T: lane holds keys 8qg + 4n + i (n, i < 4... ) of its row
    f32x4 s[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      s[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        if constexpr (FP8) {
          const bf16x8 kop = fp8x8_to_bf16(k8[n][k]);
          s[n] = mfma(kop, qop_hi[k], s[n]);
          s[n] = mfma(kop, qop_lo[k], s[n]);
        } else if constexpr (BF16) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, kraw[n][k][0]);
          s[n] = mfma(kop, qop_hi[k], s[n]);
          s[n] = mfma(kop, qop_lo[k], s[n]);
        } else {
          bf16x8 khi, klo;
          split8(kraw[n][k][0], kraw[n][k][1], khi, klo);
          s[n] = mfma(khi, qop_hi[k], s[n]);
          s[n] = mfma(khi, qop_lo[k], s[n]);
          s[n] = mfma(klo, qop_hi[k], s[n]);
        }
      }
    }
    const int gp = (qg >> 1) ? gpos[1] : gpos[0];
    const int t0 = gp + 8 * (qg & 1);  // position of key 8qg (if the group exists)
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = gp >= 0 && t0 + 4 * n + i <= tau;
        const float sc = FP8 ? s[n][i] * ksc[4 * n + i] : s[n][i];
        sv[4 * n + i] = vis ? sc : -INFINITY;
        mx = fmaxf(mx, sv[4 * n + i]);
      }
    m = rows_max(mx);
    const float mref = m == -INFINITY ? 0.f : m;
    // V of keys that are missing or after the last query token -> 0 (such
    // rows may never have been written)
    const bool partial = gpos[0] < 0 || gpos[1] < 0 || gpos[0] + kGroupTokens - 1 > pos_last ||
                         gpos[1] + kGroupTokens - 1 > pos_last;
    uint32_t keep = 0xFFu;
    if (partial) {  // wave-uniform
      keep = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) keep |= (gp >= 0 && t0 + i <= pos_last) ? (1u << i) : 0u;
    }
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float p0 = exp2f(sv[2 * k] - mref), p1 = exp2f(sv[2 * k + 1] - mref);
      l += p0 + p1;
      if constexpr (FP8) {  // the V row scale joins the probability (a kept key only)
        p0 = (keep >> (2 * k)) & 1u ? p0 * vsc[2 * k] : 0.f;
        p1 = (keep >> (2 * k + 1)) & 1u ? p1 * vsc[2 * k + 1] : 0.f;
      }
      split_pair(p0, p1, ph[k], pl[k]);
    }
    const bf16x8 pop_hi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8 pop_lo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (FP8) {
        uint2 vv = v8[nb];
        if (partial) {  // masked bytes -> +0
          uint32_t mlo = 0u, mhi = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            mlo |= (keep >> i) & 1u ? 0xFFu << (8 * i) : 0u;
            mhi |= (keep >> (4 + i)) & 1u ? 0xFFu << (8 * i) : 0u;
          }
          vv = make_uint2(vv.x & mlo, vv.y & mhi);
        }
        const bf16x8 vop = fp8x8_to_bf16(vv);
        o[nb] = mfma(vop, pop_hi, o[nb]);
        o[nb] = mfma(vop, pop_lo, o[nb]);
      } else if constexpr (BF16) {
        const uint4 vv = partial ? keep_bf16(vraw[nb][0], keep) : vraw[nb][0];
        const bf16x8 vop = __builtin_bit_cast(bf16x8, vv);
        o[nb] = mfma(vop, pop_hi, o[nb]);
        o[nb] = mfma(vop, pop_lo, o[nb]);
      } else {
        uint4 v0v = vraw[nb][0], v1v = vraw[nb][1];
        if (partial) {
          v0v = make_uint4(keep & 1u ? v0v.x : 0u, keep & 2u ? v0v.y : 0u, keep & 4u ? v0v.z : 0u,
                           keep & 8u ? v0v.w : 0u);
          v1v = make_uint4(keep & 16u ? v1v.x : 0u, keep & 32u ? v1v.y : 0u,
                           keep & 64u ? v1v.z : 0u, keep & 128u ? v1v.w : 0u);
        }
        bf16x8 vhi, vlo;
        split8(v0v, v1v, vhi, vlo);
        o[nb] = mfma(vhi, pop_hi, o[nb]);
        o[nb] = mfma(vhi, pop_lo, o[nb]);
        o[nb] = mfma(vlo, pop_hi, o[nb]);
      }
    }
  }
  // ---- merge the four waves: lane (rl, qg) holds O^T[dim 16nb + 4qg + i][row rl]
  if (qg == 0) sh.mw[wave][rl] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(sh.mw[0][rl], sh.mw[1][rl]), fmaxf(sh.mw[2][rl], sh.mw[3][rl]));
  const float f = M == -INFINITY ? 0.f : exp2f(m - M);
  l = rows_sum(l) * f;
  if (qg == 0) sh.lw[wave][rl] = l;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    *reinterpret_cast<float4*>(&sh.ob[wave][rl][16 * nb + 4 * qg]) =
        make_float4(o[nb][0] * f, o[nb][1] * f, o[nb][2] * f, o[nb][3] * f);
  __syncthreads();
  // ---- this split's partial of each query row: thread -> (row, 8 dims)
  {
    constexpr int TPR = 256 / kColRows;  // threads per row
    constexpr int EPT = D / TPR;         // dims per thread (8 or 4)
    const int r = tid / TPR, e0 = (tid % TPR) * EPT;
    const int gr = cb * kColRows + r;
    const int ri = split + record_base(a, lp);  // < n_splits for lists hga_route can write
    if (gr < n_rows && ri < args.n_splits) {
      const int tq = gr / HG, hh = gr % HG;
      float* rec = a.part + ((size_t)(unit * a.lq + tq) * args.n_splits + ri) * part_floats<D, HG>();
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        float4 acc = *reinterpret_cast<const float4*>(&sh.ob[0][r][e0 + e]);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float4 x = *reinterpret_cast<const float4*>(&sh.ob[w][r][e0 + e]);
          acc.x += x.x;
          acc.y += x.y;
          acc.z += x.z;
          acc.w += x.w;
        }
        *reinterpret_cast<float4*>(rec + part_head<HG>() + hh * D + e0 + e) = acc;
      }
      if (tid % TPR == 0) {
        rec[hh] = fmaxf(fmaxf(sh.mw[0][r], sh.mw[1][r]), fmaxf(sh.mw[2][r], sh.mw[3][r]));
        rec[HG + hh] = sh.lw[0][r] + sh.lw[1][r] + sh.lw[2][r] + sh.lw[3][r];
      }
    }
  }
}

template <int D, int HG, bool BF16, bool FP8 = false>
__global__ __launch_bounds__(256) void attend_decode_kernel(AttendArgs args) {
  decode_split<D, HG, BF16, FP8>(args, blockIdx.x, blockIdx.y, blockIdx.z);
}

// The host tier's one-launch front: workgroups [0, n_win) are the window
// part's attention splits (linearised split-fastest over the window grid),
// the rest a persistent gather of the routed groups from the pinned host
// pool into the working set.  The copy workgroups wait on PCIe most of the
// time, so the window attention runs beside the transfer instead of before
// or after it.
template <int D, int HG, bool BF16, bool FP8 = false>
__global__ __launch_bounds__(256) void tier_front_kernel(AttendArgs win, int win_x, int win_y, int n_win,
                                                         GatherArgs g, int n_items) {
  const int wg = blockIdx.x;
  if (wg >= n_win) {
    gather_items(g, n_items, wg - n_win, gridDim.x - n_win);
    return;
  }
  decode_split<D, HG, BF16, FP8>(win, wg % win_x, (wg / win_x) % win_y, wg / (win_x * win_y));
}

template <int D, int HG>
static void launch_decode_dh(const AttendArgs& x, dim3 grid, hipStream_t st) {
  if constexpr (D == 128) {
    if (x.cfg.pool8) {
      hipLaunchKernelGGL((attend_decode_kernel<D, HG, true, true>), grid, dim3(256), 0, st, x);
      return;
    }
  }
  if (x.cfg.dtype == HGA_BF16)
    hipLaunchKernelGGL((attend_decode_kernel<D, HG, true>), grid, dim3(256), 0, st, x);
  else
    hipLaunchKernelGGL((attend_decode_kernel<D, HG, false>), grid, dim3(256), 0, st, x);
}

template <int D>
static void launch_decode_d(const AttendArgs& x, dim3 grid, hipStream_t st) {
  switch (x.cfg.lhg) {
    case 1: launch_decode_dh<D, 1>(x, grid, st); break;
    case 2: launch_decode_dh<D, 2>(x, grid, st); break;
    case 4: launch_decode_dh<D, 4>(x, grid, st); break;
    default: launch_decode_dh<D, 8>(x, grid, st); break;
  }
}

template <int D, int HG>
static void launch_front_dh(const AttendArgs& x, int gx, int gy, int n_win, const GatherArgs& g,
                            int n_items, int n_gwg, hipStream_t st) {
  const dim3 grid(n_win + n_gwg);
  if constexpr (D == 128) {
    if (x.cfg.pool8) {
      hipLaunchKernelGGL((tier_front_kernel<D, HG, true, true>), grid, dim3(256), 0, st, x, gx, gy,
                         n_win, g, n_items);
      return;
    }
  }
  if (x.cfg.dtype == HGA_BF16)
    hipLaunchKernelGGL((tier_front_kernel<D, HG, true>), grid, dim3(256), 0, st, x, gx, gy, n_win, g, n_items);
  else
    hipLaunchKernelGGL((tier_front_kernel<D, HG, false>), grid, dim3(256), 0, st, x, gx, gy, n_win, g, n_items);
}

template <int D>
static void launch_front_d(const AttendArgs& x, int gx, int gy, int n_win, const GatherArgs& g,
                           int n_items, int n_gwg, hipStream_t st) {
  switch (x.cfg.lhg) {
    case 1: launch_front_dh<D, 1>(x, gx, gy, n_win, g, n_items, n_gwg, st); break;
    case 2: launch_front_dh<D, 2>(x, gx, gy, n_win, g, n_items, n_gwg, st); break;
    case 4: launch_front_dh<D, 4>(x, gx, gy, n_win, g, n_items, n_gwg, st); break;
    default: launch_front_dh<D, 8>(x, gx, gy, n_win, g, n_items, n_gwg, st); break;
  }
}

void launch_tier_front(const AttendArgs& x, int win_splits, const GatherArgs& g, int n_items,
                       hipStream_t st) {
  const int ncb = (x.cfg.lhg * x.a.lq + kColRows - 1) / kColRows;
  const int gx = win_splits, gy = x.cfg.lists;
  const int n_win = gx * gy * x.a.B * ncb;
  const int n_gwg = n_items < kGatherWgs ? n_items : kGatherWgs;
  if (x.cfg.d == 128) launch_front_d<128>(x, gx, gy, n_win, g, n_items, n_gwg, st);
  else launch_front_d<64>(x, gx, gy, n_win, g, n_items, n_gwg, st);
}

void launch_decode(const AttendArgs& x, hipStream_t st) {
  const int ncb = (x.cfg.lhg * x.a.lq + kColRows - 1) / kColRows;
  const dim3 grid(x.grid_splits, x.cfg.lists, x.a.B * ncb);
  if (x.cfg.d == 128) launch_decode_d<128>(x, grid, st);
  else launch_decode_d<64>(x, grid, st);
}

}  // namespace hga
