// Pool append and RoPE-aware chunk/group key summaries.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 3: summaries
// come from the projected keys with no new layers; high-frequency RoPE pairs
// are rotated per token and then averaged, low-frequency pairs are averaged
// raw and then rotated to the span's representative position (taken as the
// midpoint a + (n-1)/2).  Item 4: the pool keeps the exact token keys, here
// stored already rotated and rounded once to the pool dtype, and the exact
// values, stored per 16-token group as a transposed [d][16] block (the layout
// in which the attention kernels feed V to the matrix cores).
//
// One workgroup per (chunk overlapping the range, KV head, sequence).  256
// threads = P pairs x S token slices (P = d/2).  Each thread loads its pair
// for all tokens of its slice at once, then rotates them in fp64 (fp64 vector
// math runs at the fp32 non-packed rate on gfx950), stepping the angle by one
// fp64 rotation per token from a single sincos, writes the rounded pool rows
// and keeps fp64 slice sums.  Slices are then combined through LDS into the
// group and chunk summaries (fp32 stores).
#include "hga_internal.h"

namespace hga {

struct BuildArgs {
  KCfg cfg;
  const void* k_raw;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  float* chunk_sum;
  float* group_sum;
  int pos0, n_tok, pool_cap, max_chunks, B;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void build_kernel(BuildArgs a) {
  constexpr int P = D / 2;               // pairs
  constexpr int S = 256 / P;             // token slices
  constexpr int TS = kChunk / S;         // tokens per slice
  constexpr int SPG = kGroupTokens / TS; // slices per group
  using T = typename std::conditional<BF16, uint16_t, float>::type;

  __shared__ double part[S][P][2];

  const int tid = threadIdx.x;
  const int j = tid % P, s = tid / P;
  const int h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.cfg.hkv + h;
  const int chunk = a.pos0 / kChunk + blockIdx.x;
  const int c0 = chunk * kChunk;
  const int lo = a.pos0, hi = a.pos0 + a.n_tok;
  const bool complete = c0 >= lo && c0 + kChunk <= hi;
  const bool hf = (a.cfg.hf_mask >> j) & 1ull;
  const double w = a.cfg.omega[j];

  const T* kr = static_cast<const T*>(a.k_raw) + (size_t)unit * a.n_tok * D;
  const T* vr = static_cast<const T*>(a.v_new) + (size_t)unit * a.n_tok * D;
  T* kp = static_cast<T*>(a.k_pool) + (size_t)unit * a.pool_cap * D;
  T* vp = static_cast<T*>(a.v_pool) + (size_t)unit * a.pool_cap * D;

  // every load of this thread first (TS tokens of pair j), unconditionally
  // from a clamped in-range row so that they are all in flight together;
  // rows outside [lo, hi) are loaded but not used
  T xa[TS], xb[TS], ya[TS], yb[TS];
  const T* vsrc = a.k_pool ? vr : kr;
#pragma unroll
  for (int i = 0; i < TS; ++i) {
    int r = c0 + s * TS + i - lo;
    r = r < 0 ? 0 : (r >= a.n_tok ? a.n_tok - 1 : r);
    const size_t row = (size_t)r * D;
    xa[i] = kr[row + j];
    xb[i] = kr[row + j + P];
    ya[i] = vsrc[row + j];
    yb[i] = vsrc[row + j + P];
  }
  // angles of consecutive positions by rotation: (cos, sin)(p w) from
  // (cos, sin)(p0 w) and (cos, sin)(w) in fp64 (error ~1e-16 per step)
  const int p_first = c0 + s * TS;
  double cs, sn, cd, sd;
  rope_cs((double)p_first, w, &cs, &sn);
  sincos(w, &sd, &cd);
  double sa = 0.0, sb = 0.0;
#pragma unroll
  for (int i = 0; i < TS; ++i) {
    const int p = p_first + i;
    if (p >= lo && p < hi) {
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
      if (a.k_pool) {
        const size_t prow = (size_t)p * D;
        if constexpr (BF16) {
          kp[prow + j] = f64_to_bf16_rne(ra);
          kp[prow + j + P] = f64_to_bf16_rne(rb);
        } else {
          kp[prow + j] = (float)ra;
          kp[prow + j + P] = (float)rb;
        }
        // V: each 16-token group is stored transposed, a [D][16] block
        const size_t vcol = (size_t)(p / kGroupTokens) * D * kGroupTokens + p % kGroupTokens;
        vp[vcol + (size_t)j * kGroupTokens] = ya[i];
        vp[vcol + (size_t)(j + P) * kGroupTokens] = yb[i];
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
  if (!complete || !a.chunk_sum) return;  // uniform across the workgroup

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
      rope_cs((double)(c0 + s * kGroupTokens) + 0.5 * (kGroupTokens - 1), w, &cs, &sn);
      const double ra = ga * cs - gb * sn, rb = ga * sn + gb * cs;
      ga = ra;
      gb = rb;
    }
    float* gs = a.group_sum + ((size_t)unit * a.max_chunks * kGroups + (size_t)chunk * kGroups + s) * D;
    gs[j] = (float)ga;
    gs[j + P] = (float)gb;
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
      rope_cs((double)c0 + 0.5 * (kChunk - 1), w, &cs, &sn);
      const double ra = ca * cs - cb * sn, rb = ca * sn + cb * cs;
      ca = ra;
      cb = rb;
    }
    float* cs_ = a.chunk_sum + ((size_t)unit * a.max_chunks + chunk) * D;
    cs_[j] = (float)ca;
    cs_[j + P] = (float)cb;
  }
}

hipError_t launch_build(const KCfg& cfg, int B, const void* k_raw, const void* v_new, int pos0,
                        int n_tok, void* k_pool, void* v_pool, int pool_cap, float* chunk_sum,
                        float* group_sum, int max_chunks, hipStream_t st) {
  BuildArgs a{cfg, k_raw, v_new, k_pool, v_pool, chunk_sum, group_sum, pos0, n_tok, pool_cap,
              max_chunks, B};
  const int first = pos0 / kChunk, last = (pos0 + n_tok - 1) / kChunk;
  dim3 grid(last - first + 1, cfg.hkv, B);
  const bool bf = cfg.dtype == HGA_BF16;
  if (cfg.d == 128) {
    if (bf) hipLaunchKernelGGL((build_kernel<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((build_kernel<128, false>), grid, dim3(256), 0, st, a);
  } else {
    if (bf) hipLaunchKernelGGL((build_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((build_kernel<64, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hga
