// Exact softmax attention over the selected token K/V, chunked-prefill shape:
// 16..64 query tokens of one chunk against the selected groups, on the
// matrix cores.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4: after
// routing, the output is softmax attention over the exact token K/V of the
// selected set; the "Experimentele Resultaten" section reports the prefill speed-up
// of fusing this step.  Within the query's own chunk a key at position p is
// visible to query token tau only if p <= tau; every routed and window key
// precedes the chunk and is visible to all of its tokens.
//
// Work split: grid = (splits of 8 selected groups, query head, sequence),
// 256 threads.  Wave w owns query tokens 16w .. 16w+15 of the chunk; all four
// waves share the split's 128 keys, staged once in LDS.
//
// Contractions (v_mfma_f32_16x16x32_bf16, fp32 accumulate):
//   S^T = K Q^T   A = 16 keys x 32 dims of K (LDS, bf16 as stored in the
//                 pool), B = the rotated query (bf16 hi + lo parts, two
//                 products), C = 16 keys x 16 query rows: each lane holds 4
//                 keys of one query row, so the row statistics of the online
//                 softmax reduce over the 4 lanes of a column (permlane swaps)
//   O^T += V^T P^T  A = 16 dims x 32 keys of V (LDS, stored transposed),
//                 B = the probabilities of the lane's own S^T entries (bf16 hi
//                 + lo), in the key order in which S^T left them: no data
//                 moves between the two products.
// The hi/lo split (x = hi + lo, both bf16) carries 16 significant bits of the
// query and of the probabilities; K and V enter unrounded (they are bf16), so
// the products carry about 2^-17 relative error before fp32 accumulation.
//
// LDS (64 KiB): the split's K rows, 16-byte chunks XOR-swizzled by key, and
// V^T rows of 128 keys (copied from the pool's transposed group blocks),
// 8-byte units XOR-swizzled by dim, so neither the
// staging writes nor the operand reads conflict on banks.  The query needs no
// staging: each lane's QK^T operand holds both halves of its RoPE pairs.
//
// The result of each split is a partial (running max m in log2 units, sum l,
// unnormalised o) per query token in the decode kernel's layout; the merge
// kernel of the decode path combines the splits exactly.
#include "hga_attend_common.h"

namespace hga {

constexpr int kSplitKeys = kSplitGroups * kGroupTokens;    // 128 keys per split

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// x -> (hi, lo) bf16 bit patterns with x ~= hi + lo.
__device__ __forceinline__ void split_hi_lo(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne_bits(x);
  lo = bf16_rne_bits(x - __uint_as_float(hi << 16));
}

template <int D, int HG>
__global__ __launch_bounds__(256) void attend_prefill_kernel(AttendArgs args) {
  static_assert(D == 128, "staging maps assume 16 chunks of 16 bytes per key row");
  constexpr int KS = D / 32;              // k-steps of the QK^T contraction
  constexpr int NB = D / 16;              // 16-dim blocks of the output
  constexpr int CH = D / 8;               // 16-byte chunks per key row
  __shared__ __align__(16) uint16_t ks[kSplitKeys * D];   // [128 keys][D], swizzled
  __shared__ __align__(16) uint16_t vt[D * kSplitKeys];   // [D][128 keys], swizzled

  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sp = blockIdx.x, qh = blockIdx.y, b = blockIdx.z;
  const int kvh = qh / HG, hj = qh % HG;
  const int unit = b * c.hkv + kvh;
  const int rl = lane & 15, qg = lane >> 4;  // C-layout column (query row) and row group
  const int row = wave * 16 + rl;            // query token of this lane
  const int pos0 = a.q_pos0[b];
  const int n_sel = a.n_sel[unit];
  const int* sel = a.sel + (size_t)unit * a.max_sel;
  const int v0 = sp * kSplitGroups;
  int sel_spec[kSplitGroups];
#pragma unroll
  for (int g = 0; g < kSplitGroups; ++g) {
    const int v = v0 + g;
    sel_spec[g] = sel[v < a.max_sel ? v : a.max_sel - 1];
  }
  // The lane's B operand of S^T = K Q^T is its query row at dims 32k + 8qg +
  // 0..7 (k < 4): both halves of the RoPE pairs j = 8qg + i and 32 + 8qg + i,
  // so the lane rotates its own operand.  Raw dims of the row, read now.
  uint4 qraw[KS];
  {
    const int tq = row < a.lq ? row : a.lq - 1;
    const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + ((size_t)(b * c.hq + qh) * a.lq + tq) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) qraw[k] = *reinterpret_cast<const uint4*>(qsrc + 32 * k + 8 * qg);
  }

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    bad = lp.n_routed < 0;
  }
  if (bad) return;  // the merge kernel writes NaN for this unit
  const int n_part = part_count(a.part_sel, lp, n_sel);
  if (v0 >= n_part) return;  // an empty split: the merge kernel skips it
  const int pos_last = pos0 + a.lq - 1;

  // ---- the split's groups: source rows and first positions (-1: no group)
  int gpos[kSplitGroups];
  size_t gbase[kSplitGroups];
  {
    const int max_gid = a.src_cap / kGroupTokens - 1;
#pragma unroll
    for (int g = 0; g < kSplitGroups; ++g) {
      const int v = v0 + g;
      const int slot = part_slot(a.part_sel, lp, v < n_part ? v : v0);
      int gid = a.part_sel == HGA_PART_ALL ? sel_spec[g] : sel[slot];
      const bool in_range = gid >= 0 && (a.src_layout == HGA_SRC_WORKING_SET || gid <= max_gid);
      gpos[g] = (v < n_part && in_range) ? gid * kGroupTokens : -1;
      gid = gid < 0 ? 0 : (gid > max_gid ? max_gid : gid);
      gbase[g] = a.src_layout == HGA_SRC_WORKING_SET
                     ? ((size_t)unit * a.max_sel + slot) * kGroupTokens * D
                     : ((size_t)unit * a.src_cap + (size_t)gid * kGroupTokens) * D;
    }
  }
  // ---- every K/V load of the split, issued before any is used (clamped
  // addresses for missing groups; their rows are masked or zeroed below)
  //   K: iteration it loads group it, thread = (row tid/16, chunk tid%16)
  //   V: iteration it loads group it's V^T block ([D][16], as the pool stores
  //      it), thread = (dim tid/2, tokens 8*(tid%2) .. +7)
  uint4 kraw[kSplitGroups];
#pragma unroll
  for (int it = 0; it < kSplitGroups; ++it)
    kraw[it] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + gbase[it] +
                                               (size_t)(tid / CH) * D + (tid % CH) * 8);
  uint4 vraw[kSplitGroups];
#pragma unroll
  for (int it = 0; it < kSplitGroups; ++it)
    vraw[it] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + gbase[it] +
                                               (size_t)(tid >> 1) * kGroupTokens + 8 * (tid & 1));

  // ---- rotated, pre-scaled query of the lane's row at tau = pos0 + row:
  // the angle tau * omega_j is formed in fp64 as a fraction of a turn and
  // reduced exactly to [-1/2, 1/2]; sin and cos of the reduced turn run in
  // fp32 (v_sin_f32 / v_cos_f32 take turns), within ~1e-6 rad.  The result
  // is split into bf16 hi + lo operands.
  bf16x8 qop_hi[KS], qop_lo[KS];
  {
    const double tau_d = (double)(pos0 + row);
    uint32_t hi[KS][4], lo[KS][4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // pairs j = 32*half + 8qg + i
      const uint32_t wx[4] = {qraw[half].x, qraw[half].y, qraw[half].z, qraw[half].w};
      const uint32_t wy[4] = {qraw[half + 2].x, qraw[half + 2].y, qraw[half + 2].z, qraw[half + 2].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = 32 * half + 8 * qg + i;
        const double turns = tau_d * (c.omega[j] * 0.15915494309189533577);
        const float fr = (float)(turns - rint(turns));
        const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
        const float x = __uint_as_float((i & 1) ? (wx[i >> 1] & 0xFFFF0000u) : (wx[i >> 1] << 16));
        const float y = __uint_as_float((i & 1) ? (wy[i >> 1] & 0xFFFF0000u) : (wy[i >> 1] << 16));
        const float rx = (x * cs - y * sn) * c.qscale_log2;
        const float ry = (x * sn + y * cs) * c.qscale_log2;
        uint32_t hx, lx, hy, ly;
        split_hi_lo(rx, hx, lx);
        split_hi_lo(ry, hy, ly);
        if (i & 1) {
          hi[half][i >> 1] |= hx << 16; lo[half][i >> 1] |= lx << 16;
          hi[half + 2][i >> 1] |= hy << 16; lo[half + 2][i >> 1] |= ly << 16;
        } else {
          hi[half][i >> 1] = hx; lo[half][i >> 1] = lx;
          hi[half + 2][i >> 1] = hy; lo[half + 2][i >> 1] = ly;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qop_hi[k] = __builtin_bit_cast(bf16x8, make_uint4(hi[k][0], hi[k][1], hi[k][2], hi[k][3]));
      qop_lo[k] = __builtin_bit_cast(bf16x8, make_uint4(lo[k][0], lo[k][1], lo[k][2], lo[k][3]));
    }
  }

  // ---- K rows (chunk ch of key at chunk ch ^ (key % CH)) and V^T (the
  // 8-byte unit u of dim row r at unit u ^ (r % 32)); V of a key that is
  // missing or lies after the last query token is stored as zero
#pragma unroll
  for (int it = 0; it < kSplitGroups; ++it) {
    const int key = it * kGroupTokens + tid / CH, ch = tid % CH;
    *reinterpret_cast<uint4*>(ks + key * D + (ch ^ (key % CH)) * 8) = kraw[it];
  }
  {
    const int dim = tid >> 1, hf = tid & 1;
#pragma unroll
    for (int it = 0; it < kSplitGroups; ++it) {
      const int gp = gpos[it];
      uint32_t keep = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) keep |= (gp >= 0 && gp + 8 * hf + i <= pos_last) ? (1u << i) : 0u;
      const uint4 x = keep_bf16(vraw[it], keep);
      const int u0 = 4 * it + 2 * hf;  // 8-byte unit of key 16*it + 8*hf
      *reinterpret_cast<uint2*>(vt + dim * kSplitKeys + ((u0 ^ (dim & 31)) * 4)) = make_uint2(x.x, x.y);
      *reinterpret_cast<uint2*>(vt + dim * kSplitKeys + (((u0 + 1) ^ (dim & 31)) * 4)) = make_uint2(x.z, x.w);
    }
  }
  __syncthreads();
  if (wave * 16 >= a.lq) return;  // no query rows in this wave

  const int tau = pos0 + row;
  f32x4 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int t = 0; t < kSplitGroups / 2; ++t) {
    const int ga = gpos[2 * t], gb = gpos[2 * t + 1];
    if (ga < 0 && gb < 0) continue;  // uniform
    f32x4 s[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      s[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = 32 * t + 16 * n + rl;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const bf16x8 kop = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(ks + key * D + (((4 * k + qg) ^ (key % CH)) * 8)));
        s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop_hi[k], s[n], 0, 0, 0);
        s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop_lo[k], s[n], 0, 0, 0);
      }
    }
    // this lane: keys 32t + 16n + 4qg + i of query row `row`
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int gp = n ? gb : ga;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = gp >= 0 && gp + 4 * qg + i <= tau;
        sv[4 * n + i] = vis ? s[n][i] : -INFINITY;
        tmax = fmaxf(tmax, sv[4 * n + i]);
      }
    }
    tmax = rows_max(tmax);
    const float mn = fmaxf(m, tmax);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float al = exp2f(m - mref);
    l *= al;
#pragma unroll
    for (int n = 0; n < NB; ++n) o[n] *= al;
    m = mn;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = exp2f(sv[2 * k] - mref), p1 = exp2f(sv[2 * k + 1] - mref);
      l += p0 + p1;
      uint32_t h0, l0, h1, l1;
      split_hi_lo(p0, h0, l0);
      split_hi_lo(p1, h1, l1);
      ph[k] = h0 | (h1 << 16);
      pl[k] = l0 | (l1 << 16);
    }
    const bf16x8 pop_hi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8 pop_lo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int r = 16 * n + rl;  // dim
      const uint2 va = *reinterpret_cast<const uint2*>(vt + r * kSplitKeys + (((8 * t + qg) ^ (r & 31)) * 4));
      const uint2 vb = *reinterpret_cast<const uint2*>(vt + r * kSplitKeys + (((8 * t + 4 + qg) ^ (r & 31)) * 4));
      const bf16x8 vop = __builtin_bit_cast(bf16x8, make_uint4(va.x, va.y, vb.x, vb.y));
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi, o[n], 0, 0, 0);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo, o[n], 0, 0, 0);
    }
  }
  l = rows_sum(l);
  const int ri = sp + record_base(a, lp);  // < n_splits for lists hga_route can write
  if (row < a.lq && ri < args.n_splits) {
    float* rec = a.part + ((size_t)(unit * a.lq + row) * args.n_splits + ri) * part_floats<D, HG>();
    if (qg == 0) {
      rec[hj] = m;
      rec[HG + hj] = l;
    }
    float* orow = rec + part_head<HG>() + hj * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      *reinterpret_cast<float4*>(orow + 16 * n + 4 * qg) = make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
  }
}

void launch_prefill(const AttendArgs& x, hipStream_t st) {
  const dim3 grid(x.grid_splits, x.cfg.hq, x.a.B);
  switch (x.cfg.hg) {
    case 1: hipLaunchKernelGGL((attend_prefill_kernel<128, 1>), grid, dim3(256), 0, st, x); break;
    case 2: hipLaunchKernelGGL((attend_prefill_kernel<128, 2>), grid, dim3(256), 0, st, x); break;
    case 4: hipLaunchKernelGGL((attend_prefill_kernel<128, 4>), grid, dim3(256), 0, st, x); break;
    default: hipLaunchKernelGGL((attend_prefill_kernel<128, 8>), grid, dim3(256), 0, st, x); break;
  }
}

}  // namespace hga
