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
//                 keys of one query row, so the row statistics of the
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
// V^T rows of 128 keys (copied from the pool's transposed group blocks).  A
// V^T row keeps each 32-key tile in the order of the S^T entries: chunk qg of
// the tile holds keys 4qg + 0..3 and 16 + 4qg + 0..3, so one 16-byte read is
// a lane's whole A operand of O^T; chunks are XOR-swizzled by dim.  Neither
// the staging writes nor the operand reads conflict on banks.  The query
// needs no staging: each lane's QK^T operand holds both halves of its RoPE
// pairs.
//
// Softmax in two passes over registers: a split has 128 keys, so a lane's 32
// scores stay in registers; the row maximum is taken once, then the
// probabilities, then O^T.  The partial carries that maximum (no online
// rescaling inside a split).
//
// The result of each split is a partial (max m in log2 units, sum l,
// unnormalised o) per query token in the decode kernel's layout; the merge
// kernel of the decode path combines the splits exactly.
#include "hga_attend_common.h"

namespace hga {

constexpr int kSplitKeys = kSplitGroups * kGroupTokens;    // 128 keys per split

template <int D, int HG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attend_prefill_kernel(AttendArgs args) {
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
      for (int w = 0; w < 4; ++w) {  // pairs i = 2w, 2w + 1: one packed register each
        float rx[2], ry[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = 32 * half + 8 * qg + 2 * w + e;
          const double turns = tau_d * (c.omega[j] * 0.15915494309189533577);
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

  // ---- K rows (chunk ch of key at chunk ch ^ (key % CH)) and V^T (tile
  // order as above, chunk c of dim row r at c ^ (r % 16)); V of a key that is
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
      // keys 16*(it%2) + 8hf + 0..7 of tile it/2: column-group qg = 2hf and
      // 2hf + 1, half it%2 of their chunks
      const int c0 = 4 * (it >> 1) + 2 * hf, h = 4 * (it & 1);
      *reinterpret_cast<uint2*>(vt + dim * kSplitKeys + ((c0 ^ (dim & 15)) * 8) + h) = make_uint2(x.x, x.y);
      *reinterpret_cast<uint2*>(vt + dim * kSplitKeys + (((c0 + 1) ^ (dim & 15)) * 8) + h) = make_uint2(x.z, x.w);
    }
  }
  __syncthreads();
  if (wave * 16 >= a.lq) return;  // no query rows in this wave

  const int tau = pos0 + row;
  constexpr int NT = kSplitGroups / 2;  // tiles of 32 keys (two 16-key blocks)
  // ---- pass 1: S^T of all 128 keys, kept in registers.  Tile t, block n,
  // k-step k: A = keys 32t + 16n + 0..15 (this lane: key rl) at dims 32k +
  // 8qg + 0..7, chunk index swizzled by key % 16 = rl; B = the query (hi and
  // lo products into one accumulator).
  // The operand reads of tile t + 1 are issued before the products of tile
  // t (scheduling barriers keep that order), so LDS latency hides under the
  // matrix-core work.
  auto load_k = [&](int t, bf16x8 (&kop)[2][KS]) {
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int k = 0; k < KS; ++k)
        kop[n][k] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(ks + (32 * t + 16 * n + rl) * D + (((4 * k + qg) ^ rl) * 8)));
  };
  f32x4 s[NT][2];
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
  // V^T operands of tile t: dims 16n + 0..15 (this lane: dim 16n + rl) at
  // the lane's 8 keys of the tile, one 16-byte chunk of the V^T row
  auto load_v = [&](int t, bf16x8 (&vop)[NB]) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      vop[n] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(vt + (16 * n + rl) * kSplitKeys + (((4 * t + qg) ^ rl) * 8)));
  };
  bf16x8 vop[2][NB];
  load_v(0, vop[0]);  // in flight during the softmax below
  __builtin_amdgcn_sched_barrier(0);
  // ---- masks and the row maximum over the split: this lane holds keys
  // 32t + 16n + 4qg + i of query row `row`; the 4 lanes of a column hold the
  // rest of the row.  A key is visible if its group is present and it does
  // not follow the query token.  With the maximum known before any
  // probability, no running rescale of o is needed.
  float tmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int gp = gpos[2 * t + n];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = gp >= 0 && gp + 4 * qg + i <= tau;
        s[t][n][i] = vis ? s[t][n][i] : -INFINITY;
        tmax = fmaxf(tmax, s[t][n][i]);
      }
    }
  const float m = rows_max(tmax);
  const float mref = m == -INFINITY ? 0.f : m;  // a row with no visible key: p = 0
  // ---- probabilities as the B operand of O^T = V^T P^T: k-slot 4n + i of
  // tile t is key 32t + 16n + 4qg + i, split into bf16 hi + lo
  float l = 0.f;
  bf16x8 pop_hi[NT], pop_lo[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = __builtin_amdgcn_exp2f(s[t][k >> 1][2 * (k & 1)] - mref);
      const float p1 = __builtin_amdgcn_exp2f(s[t][k >> 1][2 * (k & 1) + 1] - mref);
      l += p0 + p1;
      split_pair(p0, p1, ph[k], pl[k]);
    }
    pop_hi[t] = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    pop_lo[t] = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
  }
  // ---- pass 2: O^T += V^T P^T
  f32x4 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t + 1 < NT) load_v(t + 1, vop[(t + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < NB; ++n)
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t & 1][n], pop_hi[t], o[n], 0, 0, 0);
#pragma unroll
    for (int n = 0; n < NB; ++n)
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t & 1][n], pop_lo[t], o[n], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
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
