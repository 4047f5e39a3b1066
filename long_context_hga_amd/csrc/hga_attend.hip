// Exact softmax attention over the selected token K/V, decode shape.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4: after
// routing, the output is standard softmax attention over the exact token
// K/V of the selected set; no summary value enters it.
//
// Grouped-query decode is HBM-bound (per token: 512 bytes of K/V, 2*128*Hg
// FMAs), so it stays on the VALU as a wavefront-reduction kernel:
//   grid = (splits of 8 selected groups, Hkv, B*lq), 256 threads.
//   Each wave owns 2 groups (32 tokens).  A token row (d bf16 = 256 B) is
//   read by d/8 lanes, 16 bytes each, so one wave instruction reads 4 whole
//   rows (1 KiB contiguous).  Every lane keeps the rotated, pre-scaled query
//   of all Hg heads for its 8 dims in registers; the Hg partial dots are
//   summed over the row's lanes with DPP (quad_perm + row mirrors), giving
//   every lane the Hg logits of its token.  Online softmax runs per head in
//   the log2 domain with one rescale per 4 tokens, skipped when no running
//   maximum moved; P.V accumulates Hg x 8 fp32 per lane.
//   The split's row states merge through LDS into one partial (m, l, o) per
//   head; the last split of a (sequence, KV head, query token) to finish
//   merges all partials exactly (log-sum-exp) and writes fp32 output.
// The query rotation uses fp64 angle and sincos (one per pair, shared through
// LDS), so the result does not depend on position magnitude.
#include "hga_internal.h"

namespace hga {

constexpr int kSplitGroups = 8;   // selected groups per workgroup
constexpr int kWaveGroups = 2;    // groups per wave

struct AttendArgs {
  KCfg cfg;
  AttendLaunch a;
  int n_splits;
};

template <int D, int HG>
struct AttendShared {
  float qs[HG][D];
  float mbuf[4 * (64 / (D / 8))][HG];
  float obuf[4][HG][D];
  float lbuf[4][HG];
  int flag;
};

template <bool BF16>
struct Raw8 {
  uint4 u[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> ldraw(const void* base, size_t elem) {
  Raw8<BF16> r;
  if constexpr (BF16) {
    r.u[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
  } else {
    r.u[0] = *reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
    r.u[1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem + 4);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float* f) {
  if constexpr (BF16) {
    f[0] = bf16lo(r.u[0].x); f[1] = bf16hi(r.u[0].x);
    f[2] = bf16lo(r.u[0].y); f[3] = bf16hi(r.u[0].y);
    f[4] = bf16lo(r.u[0].z); f[5] = bf16hi(r.u[0].z);
    f[6] = bf16lo(r.u[0].w); f[7] = bf16hi(r.u[0].w);
  } else {
    f[0] = __uint_as_float(r.u[0].x); f[1] = __uint_as_float(r.u[0].y);
    f[2] = __uint_as_float(r.u[0].z); f[3] = __uint_as_float(r.u[0].w);
    f[4] = __uint_as_float(r.u[1].x); f[5] = __uint_as_float(r.u[1].y);
    f[6] = __uint_as_float(r.u[1].z); f[7] = __uint_as_float(r.u[1].w);
  }
}

// Virtual group index v of a part -> slot of the unit's selected list.
__device__ __forceinline__ int part_slot(int part, const ListParts& lp, int v) {
  if (part == HGA_PART_ROUTED) return lp.n_head + v;
  if (part == HGA_PART_WINDOWS) return v < lp.n_head ? v : v + lp.n_routed;
  return v;
}
__device__ __forceinline__ int part_count(int part, const ListParts& lp, int n_sel) {
  if (part == HGA_PART_ROUTED) return lp.n_routed;
  if (part == HGA_PART_WINDOWS) return lp.n_head + lp.n_tail;
  return n_sel;
}

template <int D, int HG, bool BF16>
__global__ __launch_bounds__(256) void attend_decode_kernel(AttendArgs args) {
  constexpr int P = D / 2;
  constexpr int LPR = D / 8;        // lanes per token row
  constexpr int RPS = 64 / LPR;     // rows per wave step
  constexpr int STEPS = kGroupTokens / RPS;
  constexpr int NB = kWaveGroups * STEPS;  // row loads per lane per split
  __shared__ AttendShared<D, HG> sh;

  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / a.lq, tq = blockIdx.z % a.lq;
  const int unit = b * c.hkv + h;
  const int pos0 = a.q_pos0[b];
  const int tau = pos0 + tq;
  const int n_sel = a.n_sel[unit];
  const size_t orow0 = ((size_t)(b * c.hq + h * HG) * a.lq + tq) * D;  // head hh: + hh*lq*D

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    bad = lp.n_routed < 0;
  }
  if (bad) {
    if (split == 0) {
      for (int i = tid; i < HG * D; i += 256)
        a.out[orow0 + (size_t)(i / D) * a.lq * D + i % D] = __builtin_nanf("");
      if (a.lse && tid < HG) a.lse[(size_t)(b * c.hq + h * HG + tid) * a.lq + tq] = __builtin_nanf("");
    }
    return;
  }
  const int n_part = part_count(a.part_sel, lp, n_sel);
  const int v0 = split * kSplitGroups;
  const int* sel = a.sel + (size_t)unit * a.max_sel;

  if (v0 < n_part) {
    // ---- rotated, pre-scaled query of the HG heads at tau
    if (tid < P) {
      double cs, sn;
      rope_cs((double)tau, c.omega[tid], &cs, &sn);
      for (int hh = 0; hh < HG; ++hh) {
        const size_t row = ((size_t)(b * c.hq + h * HG + hh) * a.lq + tq) * D;
        double x, y;
        if constexpr (BF16) {
          x = bf16_to_f(static_cast<const uint16_t*>(a.q)[row + tid]);
          y = bf16_to_f(static_cast<const uint16_t*>(a.q)[row + tid + P]);
        } else {
          x = static_cast<const float*>(a.q)[row + tid];
          y = static_cast<const float*>(a.q)[row + tid + P];
        }
        sh.qs[hh][tid] = (float)(x * cs - y * sn) * c.qscale_log2;
        sh.qs[hh][tid + P] = (float)(x * sn + y * cs) * c.qscale_log2;
      }
    }

    const int sub = lane % LPR, row = lane / LPR;
    // ---- issue every K/V row load of this wave up front
    Raw8<BF16> kraw[NB], vraw[NB];
    int gpos[kWaveGroups];
#pragma unroll
    for (int gi = 0; gi < kWaveGroups; ++gi) {
      const int v = v0 + wave * kWaveGroups + gi;
      gpos[gi] = -1;
      if (v < n_part) {
        const int slot = part_slot(a.part_sel, lp, v);
        const int gid = sel[slot];
        const bool in_range = gid >= 0 && (a.src_layout == HGA_SRC_WORKING_SET ||
                                           (size_t)(gid + 1) * kGroupTokens <= (size_t)a.src_cap);
        if (!in_range) continue;  // only a list not produced by hga_route gets here
        gpos[gi] = gid * kGroupTokens;
        const size_t base = a.src_layout == HGA_SRC_WORKING_SET
                                ? ((size_t)unit * a.max_sel + slot) * kGroupTokens * D
                                : ((size_t)unit * a.src_cap + (size_t)gid * kGroupTokens) * D;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          const size_t e = base + (size_t)(st * RPS + row) * D + sub * 8;
          kraw[gi * STEPS + st] = ldraw<BF16>(a.k, e);
          vraw[gi * STEPS + st] = ldraw<BF16>(a.v, e);
        }
      }
    }
    __syncthreads();
    float q[HG][8];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int i = 0; i < 8; ++i) q[hh][i] = sh.qs[hh][sub * 8 + i];

    float m[HG], l[HG], o[HG][8];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[hh][i] = 0.f;
    }

#pragma unroll
    for (int gi = 0; gi < kWaveGroups; ++gi) {
      if (gpos[gi] < 0) continue;  // wave-uniform
      float s[STEPS][HG];
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        float kf[8];
        unpack8<BF16>(kraw[gi * STEPS + st], kf);
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float acc = q[hh][0] * kf[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) acc = fmaf(q[hh][i], kf[i], acc);
          s[st][hh] = group_sum<LPR>(acc);
        }
        const int p = gpos[gi] + st * RPS + row;
        if (p > tau) {
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) s[st][hh] = -INFINITY;
        }
      }
      // one running-max update per group and lane (its STEPS tokens)
      float mnew[HG];
      bool moved = false;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float mx = m[hh];
#pragma unroll
        for (int st = 0; st < STEPS; ++st) mx = fmaxf(mx, s[st][hh]);
        mnew[hh] = mx;
        moved |= mx > m[hh];
      }
      if (__ballot(moved) != 0ull) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          const float alpha = mnew[hh] == -INFINITY ? 1.f : exp2f(m[hh] - mnew[hh]);
          l[hh] *= alpha;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[hh][i] *= alpha;
          m[hh] = mnew[hh];
        }
      }
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        float vf[8];
        unpack8<BF16>(vraw[gi * STEPS + st], vf);
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          const float mref = m[hh] == -INFINITY ? 0.f : m[hh];
          const float pw = exp2f(s[st][hh] - mref);
          l[hh] += pw;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[hh][i] = fmaf(pw, vf[i], o[hh][i]);
        }
      }
    }

    // ---- merge the 4*RPS row states of the workgroup
    if (sub == 0) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) sh.mbuf[wave * RPS + row][hh] = m[hh];
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      float M = -INFINITY;
      for (int r = 0; r < 4 * RPS; ++r) M = fmaxf(M, sh.mbuf[r][hh]);
      const float f = M == -INFINITY ? 0.f : exp2f(m[hh] - M);
      l[hh] *= f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[hh][i] *= f;
      m[hh] = M;
    }
#pragma unroll
    for (int msk = LPR; msk < 64; msk <<= 1) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        l[hh] += __shfl_xor(l[hh], msk, 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[hh][i] += __shfl_xor(o[hh][i], msk, 64);
      }
    }
    if (row == 0) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sh.obuf[wave][hh][sub * 8 + i] = o[hh][i];
        if (sub == 0) sh.lbuf[wave][hh] = l[hh];
      }
    }
    __syncthreads();
    float* part = a.part + ((size_t)(unit * a.lq + tq) * args.n_splits + split) * (HG * (D + 2));
    for (int i = tid; i < HG * D; i += 256) {
      const int hh = i / D, e = i % D;
      part[2 * HG + i] = sh.obuf[0][hh][e] + sh.obuf[1][hh][e] + sh.obuf[2][hh][e] + sh.obuf[3][hh][e];
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {  // every thread holds the workgroup max of each head
      if (tid == hh) {
        part[hh] = m[hh];
        part[HG + hh] = sh.lbuf[0][hh] + sh.lbuf[1][hh] + sh.lbuf[2][hh] + sh.lbuf[3][hh];
      }
    }
  }

  // ---- last split of this (unit, query token) merges the partials
  if (!arrive_last(a.counters + unit * a.lq + tq, args.n_splits, &sh.flag)) return;
  const int n_act = (n_part + kSplitGroups - 1) / kSplitGroups;
  const float* pbase = a.part + (size_t)(unit * a.lq + tq) * args.n_splits * (HG * (D + 2));
  for (int i = tid; i < HG * D; i += 256) {
    const int hh = i / D, e = i % D;
    float M = -INFINITY;
    for (int sp = 0; sp < n_act; ++sp) M = fmaxf(M, pbase[(size_t)sp * HG * (D + 2) + hh]);
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
      for (int sp = 0; sp < n_act; ++sp) {
        const float* pp = pbase + (size_t)sp * HG * (D + 2);
        const float f = exp2f(pp[hh] - M);
        L = fmaf(f, pp[HG + hh], L);
        acc = fmaf(f, pp[2 * HG + i], acc);
      }
    }
    a.out[orow0 + (size_t)hh * a.lq * D + e] = L > 0.f ? acc / L : 0.f;
    if (a.lse && e == 0)
      a.lse[(size_t)(b * c.hq + h * HG + hh) * a.lq + tq] =
          L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
  }
}

size_t attend_ws_bytes(const KCfg& cfg, int B, int lq, int max_sel) {
  const int n_splits = (max_sel + kSplitGroups - 1) / kSplitGroups;
  return (size_t)B * cfg.hkv * lq * n_splits * cfg.hg * (cfg.d + 2) * sizeof(float);
}

template <int D, int HG>
static void launch_dh(const AttendArgs& x, dim3 grid, hipStream_t st) {
  if (x.cfg.dtype == HGA_BF16)
    hipLaunchKernelGGL((attend_decode_kernel<D, HG, true>), grid, dim3(256), 0, st, x);
  else
    hipLaunchKernelGGL((attend_decode_kernel<D, HG, false>), grid, dim3(256), 0, st, x);
}

template <int D>
static void launch_d(const AttendArgs& x, dim3 grid, hipStream_t st) {
  switch (x.cfg.hg) {
    case 1: launch_dh<D, 1>(x, grid, st); break;
    case 2: launch_dh<D, 2>(x, grid, st); break;
    case 4: launch_dh<D, 4>(x, grid, st); break;
    default: launch_dh<D, 8>(x, grid, st); break;
  }
}

hipError_t launch_attend(const KCfg& cfg, const AttendLaunch& a, hipStream_t st) {
  AttendArgs x;
  x.cfg = cfg;
  x.a = a;
  x.n_splits = (a.max_sel + kSplitGroups - 1) / kSplitGroups;
  dim3 grid(x.n_splits, cfg.hkv, a.B * a.lq);
  if (cfg.d == 128) launch_d<128>(x, grid, st);
  else launch_d<64>(x, grid, st);
  return hipGetLastError();
}

}  // namespace hga
