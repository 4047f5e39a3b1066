// Device body of the pool append and the RoPE-aware chunk/group summaries,
// shared by hga_build_summaries and the fused decode step.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 3: summaries
// come from the projected keys with no new layers; high-frequency RoPE pairs
// are rotated per token and then averaged, low-frequency pairs are averaged
// raw and then rotated to the span's representative position (the midpoint
// a + (n-1)/2 by default; a + n/2 as a configured variant).
//
// 256 threads = P pairs x S token slices (P = d/2).  Each thread loads its
// pair for all tokens of its slice at once, rotates them in fp64, stepping the
// angle by one fp64 rotation per token from a single sincos, writes the
// rounded pool rows and keeps fp64 slice sums; the slices combine through LDS
// into the group and chunk summaries (fp32 stores).
#pragma once

#include "hga_internal.h"

namespace hga {

// The work of one chunk (start c0) for the tokens [lo, hi) of a unit:
// rotated keys and values of those tokens into the pool (kp, vp: the unit's
// pool bases, NULL = no append), and, if the chunk lies entirely inside
// [lo, hi), its chunk summary (cs_row) and G group summaries (gs_rows, G
// consecutive rows); NULL = no summaries.  krow(p) / vrow(p) return the raw
// key / value row of position p in [lo, hi).  stage (nullable): the chunk's
// staging rows, [C][D]; the raw key of each position in [lo, hi) is copied
// to row p - c0.  part: LDS scratch of S*P*2 doubles.  f8 (with f8.k set,
// in place of kp / vp; head_dim 128): the append writes the FP8 pool instead,
// E4M3FN codes of each rotated key row and value row with their row scales.
// Called by all 256 threads of a workgroup with uniform arguments.
struct Fp8Rows {
  uint8_t* k = nullptr;  // the unit's K codes [cap][D]
  uint8_t* v = nullptr;  // the unit's V^T codes [cap/16][D][16]
  float* ks = nullptr;   // the unit's K row scales [cap]
  float* vs = nullptr;   // the unit's V row scales [cap]
};

// The FP8 pool buffers: codes of every unit ([units][cap][D] bytes, V in
// transposed group blocks), then the row scales ([units][cap] fp32).
__device__ __forceinline__ Fp8Rows fp8_rows_of(void* k_pool, void* v_pool, int units, int cap, int d,
                                               int unit) {
  Fp8Rows r;
  const size_t codes = (size_t)units * cap * d;
  r.k = static_cast<uint8_t*>(k_pool) + (size_t)unit * cap * d;
  r.v = static_cast<uint8_t*>(v_pool) + (size_t)unit * cap * d;
  r.ks = reinterpret_cast<float*>(static_cast<uint8_t*>(k_pool) + codes) + (size_t)unit * cap;
  r.vs = reinterpret_cast<float*>(static_cast<uint8_t*>(v_pool) + codes) + (size_t)unit * cap;
  return r;
}

// One token's rows into the FP8 pool (bf16 inputs, head_dim 128), as
// build_span writes them: wave 0 rotates and quantises the key row (lane j:
// pair j, the angle stepped from the first position of the token's slice
// exactly as build_span steps it), wave 1 quantises the value row.
__device__ __forceinline__ void fp8_append_row(const KCfg& cfg, const uint16_t* kn, const uint16_t* vn,
                                            int c0, int p, Fp8Rows f8) {
  constexpr int D = 128, P = D / 2, TS = kChunk / (256 / P);
  const int wave = threadIdx.x >> 6, j = threadIdx.x & 63;
  if (wave > 1) return;
  const int ja = pair_a(cfg, j), jb = pair_b(cfg, j);
  double xa, xb;
  if (wave == 0) {
    const double w = cfg.omega[j];
    const int p_first = c0 + (p - c0) / TS * TS;
    double cs, sn, cd, sd;
    rope_cs((double)p_first, w, &cs, &sn);
    sincos_rad(w, &sd, &cd);
    for (int i = p_first; i < p; ++i) {
      const double c2 = cs * cd - sn * sd;
      sn = sn * cd + cs * sd;
      cs = c2;
    }
    const double ka = bf16_to_f(kn[ja]), kb = bf16_to_f(kn[jb]);
    xa = ka * cs - kb * sn;
    xb = ka * sn + kb * cs;
  } else {
    xa = bf16_to_f(vn[ja]);
    xb = bf16_to_f(vn[jb]);
  }
  const double sc = fp8_row_scale(wave_ext_d<true>(fmax(fabs(xa), fabs(xb))));
  const uint8_t ca = (uint8_t)fp8_code(xa / sc), cb = (uint8_t)fp8_code(xb / sc);
  if (wave == 0) {
    f8.k[(size_t)p * D + ja] = ca;
    f8.k[(size_t)p * D + jb] = cb;
    if (j == 0) f8.ks[p] = (float)sc;
  } else {
    const size_t vcol = (size_t)(p / kGroupTokens) * D * kGroupTokens + p % kGroupTokens;
    f8.v[vcol + (size_t)ja * kGroupTokens] = ca;
    f8.v[vcol + (size_t)jb * kGroupTokens] = cb;
    if (j == 0) f8.vs[p] = (float)sc;
  }
}

template <int D, bool BF16, class KRow, class VRow>
__device__ __forceinline__ void build_span(
    const KCfg& cfg, int c0, int lo, int hi, KRow krow, VRow vrow,
    typename std::conditional<BF16, uint16_t, float>::type* kp,
    typename std::conditional<BF16, uint16_t, float>::type* vp, float* cs_row, float* gs_rows,
    double* part_lds, typename std::conditional<BF16, uint16_t, float>::type* stage = nullptr,
    Fp8Rows f8 = {}) {
  constexpr int P = D / 2;               // pairs
  constexpr int S = 256 / P;             // token slices
  constexpr int TS = kChunk / S;         // tokens per slice
  constexpr int SPG = kGroupTokens / TS; // slices per group
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  double (*part)[P][2] = reinterpret_cast<double (*)[P][2]>(part_lds);

  const int tid = threadIdx.x;
  const int j = tid % P, s = tid / P;
  const bool complete = c0 >= lo && c0 + kChunk <= hi;
  const bool hf = (cfg.hf_mask >> j) & 1ull;
  const int ja = pair_a(cfg, j), jb = pair_b(cfg, j);  // dims of the pair's members
  const double w = cfg.omega[j];

  // every load of this thread first (TS tokens of pair j), unconditionally
  // from a clamped in-range row so that they are all in flight together;
  // rows outside [lo, hi) are loaded but not used
  T xa[TS], xb[TS], ya[TS], yb[TS];
#pragma unroll
  for (int i = 0; i < TS; ++i) {
    int p = c0 + s * TS + i;
    p = p < lo ? lo : (p >= hi ? hi - 1 : p);
    const T* kr = krow(p);
    const T* vr = (kp || f8.k) ? vrow(p) : kr;
    xa[i] = kr[ja];
    xb[i] = kr[jb];
    ya[i] = vr[ja];
    yb[i] = vr[jb];
  }
  // angles of consecutive positions by rotation: (cos, sin)(p w) from
  // (cos, sin)(p0 w) and (cos, sin)(w) in fp64 (error ~1e-16 per step)
  const int p_first = c0 + s * TS;
  double cs, sn, cd, sd;
  rope_cs((double)p_first, w, &cs, &sn);
  sincos_rad(w, &sd, &cd);
  double sa = 0.0, sb = 0.0;
#pragma unroll
  for (int i = 0; i < TS; ++i) {
    const int p = p_first + i;
    if (p >= lo && p < hi) {
      if (stage) {
        stage[(size_t)(p - c0) * D + ja] = xa[i];
        stage[(size_t)(p - c0) * D + jb] = xb[i];
      }
      double ka, kb;
      if constexpr (BF16) {
        ka = bf16_to_f(xa[i]);
        kb = bf16_to_f(xb[i]);
      } else {
        ka = xa[i];
        kb = xb[i];
      }
      const double ra = ka * cs - kb * sn;
      const double rb = ka * sn + kb * cs;
      if (kp) {
        const size_t prow = (size_t)p * D;
        if constexpr (BF16) {
          kp[prow + ja] = f64_to_bf16_rne(ra);
          kp[prow + jb] = f64_to_bf16_rne(rb);
        } else {
          kp[prow + ja] = (float)ra;
          kp[prow + jb] = (float)rb;
        }
        // V: each 16-token group is stored transposed, a [D][16] block
        const size_t vcol = (size_t)(p / kGroupTokens) * D * kGroupTokens + p % kGroupTokens;
        vp[vcol + (size_t)ja * kGroupTokens] = ya[i];
        vp[vcol + (size_t)jb * kGroupTokens] = yb[i];
      }
      if constexpr (D == 128 && BF16) {
        if (f8.k) {  // uniform; the wave holds the 64 pairs of this token
          const double va = bf16_to_f(ya[i]), vb = bf16_to_f(yb[i]);
          const double sk = fp8_row_scale(wave_ext_d<true>(fmax(fabs(ra), fabs(rb))));
          const double sv = fp8_row_scale(wave_ext_d<true>(fmax(fabs(va), fabs(vb))));
          const size_t prow = (size_t)p * D;
          f8.k[prow + ja] = (uint8_t)fp8_code(ra / sk);
          f8.k[prow + jb] = (uint8_t)fp8_code(rb / sk);
          const size_t vcol = (size_t)(p / kGroupTokens) * D * kGroupTokens + p % kGroupTokens;
          f8.v[vcol + (size_t)ja * kGroupTokens] = (uint8_t)fp8_code(va / sv);
          f8.v[vcol + (size_t)jb * kGroupTokens] = (uint8_t)fp8_code(vb / sv);
          if (j == 0) {
            f8.ks[p] = (float)sk;
            f8.vs[p] = (float)sv;
          }
        }
      }
      if (hf) {
        sa += ra;
        sb += rb;
      } else {
        sa += ka;
        sb += kb;
      }
    }
    const double c2 = cs * cd - sn * sd;
    sn = sn * cd + cs * sd;
    cs = c2;
  }
  if (!complete || !cs_row) return;  // uniform across the workgroup

  part[s][j][0] = sa;
  part[s][j][1] = sb;
  __syncthreads();

  // group gi = s (s < G): sum its slices
  if (s < kGroups) {
    double ga = 0.0, gb = 0.0;
    for (int q = 0; q < SPG; ++q) {
      ga += part[s * SPG + q][j][0];
      gb += part[s * SPG + q][j][1];
    }
    ga /= kGroupTokens;
    gb /= kGroupTokens;
    if (!hf) {
      double cs, sn;
      rope_cs((double)(c0 + s * kGroupTokens) + 0.5 * (kGroupTokens - 1) + cfg.rep_shift, w, &cs, &sn);
      const double ra = ga * cs - gb * sn, rb = ga * sn + gb * cs;
      ga = ra;
      gb = rb;
    }
    float* gs = gs_rows + (size_t)s * D;
    gs[ja] = (float)ga;
    gs[jb] = (float)gb;
  }
  if (s == 0) {
    double ca = 0.0, cb = 0.0;
    for (int q = 0; q < S; ++q) {
      ca += part[q][j][0];
      cb += part[q][j][1];
    }
    ca /= kChunk;
    cb /= kChunk;
    if (!hf) {
      double cs, sn;
      rope_cs((double)c0 + 0.5 * (kChunk - 1) + cfg.rep_shift, w, &cs, &sn);
      const double ra = ca * cs - cb * sn, rb = ca * sn + cb * cs;
      ca = ra;
      cb = rb;
    }
    cs_row[ja] = (float)ca;
    cs_row[jb] = (float)cb;
  }
}


}  // namespace hga
