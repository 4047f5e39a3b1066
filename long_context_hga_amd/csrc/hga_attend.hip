// Exact softmax attention over the selected token K/V, decode shape.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4: after
// routing, the output is standard softmax attention over the exact token
// K/V of the selected set; no summary value enters it.
//
// Grouped-query decode moves 512 bytes of K/V per token and KV head for
// 2*128*Hg FMAs, so it stays on the VALU as a wavefront-reduction kernel:
//   grid = (splits of 8 selected groups, Hkv, B*lq), 256 threads.
//   Each wave owns 2 groups (32 tokens).  A token row (d bf16 = 256 B) is
//   read by d/8 lanes, 16 bytes each, so one wave instruction reads 4 whole
//   rows (1 KiB contiguous).  All K/V loads of a wave are issued before any
//   is used.  Every lane keeps the rotated, pre-scaled query of the Hg heads
//   for its 8 dims in registers and forms Hg partial dot products.
//   d = 128, Hg = 8 (the grouped-query shape): the 16 lanes of a row
//   reduce-scatter the 8 partial dots with DPP (row_ror:8, half-row mirror,
//   quad permutes): each lane ends with the logit of one head, so the online
//   softmax costs one exp2 per lane and token; the 8 probabilities are
//   gathered back with 7 DPP moves for P.V.  The head held in each register
//   slot is permuted per lane (head = lane ^ {0,1,2,3,7,6,5,4}[slot]) so that
//   every reduce step is a plain DPP add.  The 4 token rows of a wave merge
//   with v_permlane16/32_swap.
//   Other shapes: every lane all-reduces the Hg dots over its row.
//   The running maximum is updated once per group (4 tokens per lane) and
//   the accumulators are rescaled only when it moved.  The split's state
//   merges through LDS into one partial (m, l, o) per head; a second kernel
//   merges the partials of all splits of a (sequence, KV head, query token)
//   exactly (log-sum-exp) and writes fp32 output.  Token rows after the
//   query position are masked, and their V (possibly never written) is
//   replaced by zeros before it meets a zero probability.
// The query rotation uses an fp64 angle and sincos (one per pair, shared
// through LDS), so the result does not depend on position magnitude.
#include "hga_attend_common.h"

namespace hga {

constexpr int kWaveGroups = 2;    // groups per wave

template <int D, int HG>
struct AttendShared {
  float qs[HG][D];
  float mrow[4 * (64 / (D / 8))][HG];  // row-state maxima (all-reduce path)
  float mw[4][HG];                     // per-wave maxima (reduce-scatter path)
  float obuf[4][HG][D];
  float lbuf[4][HG];
  float mmax[HG];
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

// Reduce-scatter layout (d = 128, Hg = 8): register slot k of a lane whose
// column index within its 8-lane half-row is i holds head i ^ kSlotMask[k].
constexpr int kSlotMask[8] = {0, 1, 2, 3, 7, 6, 5, 4};
constexpr int kDppRor8 = 0x128;
constexpr int kDppXor3 = 0x1B;  // quad_perm [3,2,1,0]

// x of head i (this lane's head) -> p[k] = x of head i ^ kSlotMask[k], from
// the lanes of the same 8-lane half-row.
__device__ __forceinline__ void gather8(float x, float* p) {
  p[0] = x;
  p[1] = dpp_f<kDppXor1>(x);
  p[2] = dpp_f<kDppXor2>(x);
  p[3] = dpp_f<kDppXor3>(x);
  p[4] = dpp_f<kDppHalfMirror>(x);
  p[5] = dpp_f<kDppXor1>(p[4]);
  p[6] = dpp_f<kDppXor2>(p[4]);
  p[7] = dpp_f<kDppXor3>(p[4]);
}

template <int D, int HG, bool BF16>
__global__ __launch_bounds__(256) void attend_decode_kernel(AttendArgs args) {
  constexpr int P = D / 2;
  constexpr int LPR = D / 8;        // lanes per token row
  constexpr int RPS = 64 / LPR;     // rows per wave step
  constexpr int STEPS = kGroupTokens / RPS;
  constexpr int NB = kWaveGroups * STEPS;  // row loads per lane per split
  constexpr bool RS = (D == 128 && HG == 8);  // reduce-scatter path
  __shared__ AttendShared<D, HG> sh;

  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / a.lq, tq = blockIdx.z % a.lq;
  const int unit = b * c.hkv + h;
  const int pos0 = a.q_pos0[b];
  const int n_sel = a.n_sel[unit];
  const int* sel = a.sel + (size_t)unit * a.max_sel;
  const int v0 = split * kSplitGroups;
  // list slots of this wave's groups when the part is the whole list: read
  // them now, in parallel with n_sel and the position
  int sel_spec[kWaveGroups];
#pragma unroll
  for (int gi = 0; gi < kWaveGroups; ++gi) {
    const int v = v0 + wave * kWaveGroups + gi;
    sel_spec[gi] = sel[v < a.max_sel ? v : a.max_sel - 1];
  }
  // raw query pair (j, j+P) of the HG heads and omega_j, read up front
  using QT = typename std::conditional<BF16, uint16_t, float>::type;
  const int jq = tid % P;
  const double wj = c.omega[jq];
  QT qx[HG], qy[HG];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    const size_t row = ((size_t)(b * c.hq + h * HG + hh) * a.lq + tq) * D;
    qx[hh] = static_cast<const QT*>(a.q)[row + jq];
    qy[hh] = static_cast<const QT*>(a.q)[row + jq + P];
  }
  const int tau = pos0 + tq;

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    bad = lp.n_routed < 0;
  }
  if (bad) return;  // the combine kernel writes NaN for this unit
  const int n_part = part_count(a.part_sel, lp, n_sel);
  if (v0 >= n_part) return;  // an empty split: the combine kernel skips it
  {
    const int sub = lane % LPR, row = lane / LPR;
    // Every K/V row load of this wave is issued before any is used.  A group
    // slot past the part's end (or a group id outside the source, which only
    // a list not produced by hga_route can hold) loads from a clamped
    // in-range address and is skipped afterwards.
    Raw8<BF16> kraw[NB], vraw[NB];
    int gpos[kWaveGroups], slots[kWaveGroups], gids[kWaveGroups];
    const int max_gid = a.src_cap / kGroupTokens - 1;
#pragma unroll
    for (int gi = 0; gi < kWaveGroups; ++gi) {
      const int v = v0 + wave * kWaveGroups + gi;
      slots[gi] = part_slot(a.part_sel, lp, v < n_part ? v : v0);
      gids[gi] = sel_spec[gi];
    }
    if (a.part_sel != HGA_PART_ALL) {  // uniform; only the parts need a second list read
#pragma unroll
      for (int gi = 0; gi < kWaveGroups; ++gi) gids[gi] = sel[slots[gi]];
    }
#pragma unroll
    for (int gi = 0; gi < kWaveGroups; ++gi) {
      const int v = v0 + wave * kWaveGroups + gi;
      int gid = gids[gi];
      const bool in_range = gid >= 0 && (a.src_layout == HGA_SRC_WORKING_SET || gid <= max_gid);
      gpos[gi] = (v < n_part && in_range) ? gid * kGroupTokens : -1;
      gid = gid < 0 ? 0 : (gid > max_gid ? max_gid : gid);
      const size_t base = a.src_layout == HGA_SRC_WORKING_SET
                              ? ((size_t)unit * a.max_sel + slots[gi]) * kGroupTokens * D
                              : ((size_t)unit * a.src_cap + (size_t)gid * kGroupTokens) * D;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        const size_t e = base + (size_t)(st * RPS + row) * D + sub * 8;
        kraw[gi * STEPS + st] = ldraw<BF16>(a.k, e);
        vraw[gi * STEPS + st] = ldraw<BF16>(a.v, e);
      }
    }
    // ---- rotated, pre-scaled query of the HG heads at tau (while the K/V
    // loads are in flight)
    if (tid < P) {
      double cs, sn;
      rope_cs((double)tau, wj, &cs, &sn);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        double x, y;
        if constexpr (BF16) {
          x = bf16_to_f(qx[hh]);
          y = bf16_to_f(qy[hh]);
        } else {
          x = qx[hh];
          y = qy[hh];
        }
        sh.qs[hh][tid] = (float)(x * cs - y * sn) * c.qscale_log2;
        sh.qs[hh][tid + P] = (float)(x * sn + y * cs) * c.qscale_log2;
      }
    }
    __syncthreads();

    if constexpr (RS) {
      // ================= reduce-scatter path (d = 128, Hg = 8)
      const int hi = sub & 7;  // this lane's head
      float q[8][8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) q[k][i] = sh.qs[hi ^ kSlotMask[k]][sub * 8 + i];
      float m = -INFINITY, l = 0.f, o[8][8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[k][i] = 0.f;

#pragma unroll
      for (int gi = 0; gi < kWaveGroups; ++gi) {
        if (gpos[gi] < 0) continue;  // wave-uniform
        float lg[STEPS];
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          float kf[8];
          unpack8<BF16>(kraw[gi * STEPS + st], kf);
          float acc[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            float t = q[k][0] * kf[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) t = fmaf(q[k][i], kf[i], t);
            acc[k] = t;
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[k] += dpp_f<kDppRor8>(acc[k]);
          float r4[4], r2[2];
#pragma unroll
          for (int k = 0; k < 4; ++k) r4[k] = acc[k] + dpp_f<kDppHalfMirror>(acc[4 + k]);
#pragma unroll
          for (int k = 0; k < 2; ++k) r2[k] = r4[k] + dpp_f<kDppXor2>(r4[2 + k]);
          const float logit = r2[0] + dpp_f<kDppXor1>(r2[1]);
          lg[st] = (gpos[gi] + st * RPS + row <= tau) ? logit : -INFINITY;
        }
        float mx = m;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) mx = fmaxf(mx, lg[st]);
        if (__ballot(mx > m) != 0ull) {
          const float al = mx == -INFINITY ? 1.f : exp2f(m - mx);
          float a8[8];
          gather8(al, a8);
          l *= al;
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) o[k][i] *= a8[k];
          m = mx;
        }
        const float mref = m == -INFINITY ? 0.f : m;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          const float pw = exp2f(lg[st] - mref);
          l += pw;
          float p8[8], vf[8];
          gather8(pw, p8);
          unpack8<BF16>(vraw[gi * STEPS + st], vf);
          if (gpos[gi] + st * RPS + row > tau) {  // a row not yet written may hold NaN
#pragma unroll
            for (int i = 0; i < 8; ++i) vf[i] = 0.f;
          }
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) o[k][i] = fmaf(p8[k], vf[i], o[k][i]);
        }
      }
      // ---- merge: workgroup max per head, rescale, sum rows, then waves
      const float mrow = rows_max(m);
      if (lane < 8) sh.mw[wave][lane] = mrow;
      __syncthreads();
      float M = fmaxf(fmaxf(sh.mw[0][hi], sh.mw[1][hi]), fmaxf(sh.mw[2][hi], sh.mw[3][hi]));
      const float f = M == -INFINITY ? 0.f : exp2f(m - M);
      float f8[8];
      gather8(f, f8);
      l = rows_sum(l * f);
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[k][i] = rows_sum(o[k][i] * f8[k]);
      if (lane < 16) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int i = 0; i < 8; ++i) sh.obuf[wave][hi ^ kSlotMask[k]][sub * 8 + i] = o[k][i];
        if (lane < 8) sh.lbuf[wave][hi] = l;
      }
      if (wave == 0 && lane < 8) sh.mmax[hi] = M;
    } else {
      // ================= all-reduce path (other shapes)
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
          if (gpos[gi] + st * RPS + row > tau) {
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) s[st][hh] = -INFINITY;
          }
        }
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
          if (gpos[gi] + st * RPS + row > tau) {  // a row not yet written may hold NaN
#pragma unroll
            for (int i = 0; i < 8; ++i) vf[i] = 0.f;
          }
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
      if (sub == 0) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) sh.mrow[wave * RPS + row][hh] = m[hh];
      }
      __syncthreads();
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float M = -INFINITY;
        for (int r = 0; r < 4 * RPS; ++r) M = fmaxf(M, sh.mrow[r][hh]);
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
      if (tid == 0) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) sh.mmax[hh] = m[hh];
      }
    }
    __syncthreads();
    // ---- this split's partial: (m, l, o) per head, published for the merge
    // layout per split: m[HG], l[HG], pad to 4, o[HG][D]
    float* part = a.part + ((size_t)(unit * a.lq + tq) * args.n_splits + split) * part_floats<D, HG>();
    for (int i = 4 * tid; i < HG * D; i += 4 * 256) {
      const int hh = i / D, e = i % D;
      float4 v;
      v.x = sh.obuf[0][hh][e] + sh.obuf[1][hh][e] + sh.obuf[2][hh][e] + sh.obuf[3][hh][e];
      v.y = sh.obuf[0][hh][e + 1] + sh.obuf[1][hh][e + 1] + sh.obuf[2][hh][e + 1] + sh.obuf[3][hh][e + 1];
      v.z = sh.obuf[0][hh][e + 2] + sh.obuf[1][hh][e + 2] + sh.obuf[2][hh][e + 2] + sh.obuf[3][hh][e + 2];
      v.w = sh.obuf[0][hh][e + 3] + sh.obuf[1][hh][e + 3] + sh.obuf[2][hh][e + 3] + sh.obuf[3][hh][e + 3];
      *reinterpret_cast<float4*>(part + part_head<HG>() + i) = v;
    }
    if (tid < HG) {
      part[tid] = sh.mmax[tid];
      part[HG + tid] = sh.lbuf[0][tid] + sh.lbuf[1][tid] + sh.lbuf[2][tid] + sh.lbuf[3][tid];
    }
  }
}

// Merge of the splits of one (sequence, KV head, query token): exact
// log-sum-exp combination of the partial (m, l, o) of every non-empty split.
// grid = B*Hkv*lq workgroups of 256 threads; thread t owns 4 consecutive
// outputs (head t*4/D), and issues all its loads (every split's m, l and
// 4 o values) before using any.
template <int D, int HG>
__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs args) {
  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / a.lq, tq = blockIdx.x % a.lq;
  const int b = unit / c.hkv, h = unit % c.hkv;
  const size_t orow0 = ((size_t)(b * c.hq + h * HG) * a.lq + tq) * D;  // head hh: + hh*lq*D
  const int i0 = 4 * tid;  // first output of this thread
  const int hh = i0 / D, e = i0 % D;
  const bool mine = i0 < HG * D;
  // every split's (m, l, 4 o values) of this thread's head is read before the
  // list length is known (splits that did not run are read but not used)
  const int ic = mine ? i0 : 0;
  const int hc = mine ? hh : 0;
  const float* pbase = a.part + (size_t)(unit * a.lq + tq) * args.n_splits * part_floats<D, HG>();
  float pm[kMaxSplits], pl[kMaxSplits];
  float4 po[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    if (sp < args.n_splits) {  // uniform
      const float* pp = pbase + (size_t)sp * part_floats<D, HG>();
      pm[sp] = pp[hc];
      pl[sp] = pp[HG + hc];
      po[sp] = *reinterpret_cast<const float4*>(pp + part_head<HG>() + ic);
    }
  }
  const int pos0 = a.q_pos0[b];
  const int n_sel = a.n_sel[unit];

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    bad = lp.n_routed < 0;
  }
  if (bad) {
    if (mine) {
      const float nan = __builtin_nanf("");
      *reinterpret_cast<float4*>(a.out + orow0 + (size_t)hh * a.lq * D + e) = make_float4(nan, nan, nan, nan);
      if (a.lse && e == 0) a.lse[(size_t)(b * c.hq + h * HG + hh) * a.lq + tq] = nan;
    }
    return;
  }
  if (!mine) return;
  const int n_part = part_count(a.part_sel, lp, n_sel);
  const int n_act = (n_part + kSplitGroups - 1) / kSplitGroups;
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < n_act) M = fmaxf(M, pm[sp]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      if (sp < n_act) {
        const float wgt = exp2f(pm[sp] - M);
        L = fmaf(wgt, pl[sp], L);
        acc.x = fmaf(wgt, po[sp].x, acc.x);
        acc.y = fmaf(wgt, po[sp].y, acc.y);
        acc.z = fmaf(wgt, po[sp].z, acc.z);
        acc.w = fmaf(wgt, po[sp].w, acc.w);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(a.out + orow0 + (size_t)hh * a.lq * D + e) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse && e == 0)
    a.lse[(size_t)(b * c.hq + h * HG + hh) * a.lq + tq] =
        L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

size_t attend_ws_bytes(const KCfg& cfg, int B, int lq, int max_sel) {
  const int n_splits = (max_sel + kSplitGroups - 1) / kSplitGroups;
  const int pf = ((2 * cfg.hg + 3) / 4 * 4) + cfg.hg * cfg.d;
  return (size_t)B * cfg.hkv * lq * n_splits * pf * sizeof(float);
}

template <int D, int HG>
static void launch_dh(const AttendArgs& x, dim3 grid, hipStream_t st) {
  if (x.cfg.dtype == HGA_BF16)
    hipLaunchKernelGGL((attend_decode_kernel<D, HG, true>), grid, dim3(256), 0, st, x);
  else
    hipLaunchKernelGGL((attend_decode_kernel<D, HG, false>), grid, dim3(256), 0, st, x);
  hipLaunchKernelGGL((attend_combine_kernel<D, HG>), dim3(x.a.B * x.cfg.hkv * x.a.lq), dim3(256), 0,
                     st, x);
}

template <int D>
static void launch_combine_d(const AttendArgs& x, dim3 grid, hipStream_t st) {
  switch (x.cfg.hg) {
    case 1: hipLaunchKernelGGL((attend_combine_kernel<D, 1>), grid, dim3(256), 0, st, x); break;
    case 2: hipLaunchKernelGGL((attend_combine_kernel<D, 2>), grid, dim3(256), 0, st, x); break;
    case 4: hipLaunchKernelGGL((attend_combine_kernel<D, 4>), grid, dim3(256), 0, st, x); break;
    default: hipLaunchKernelGGL((attend_combine_kernel<D, 8>), grid, dim3(256), 0, st, x); break;
  }
}

static void launch_combine(const AttendArgs& x, hipStream_t st) {
  const dim3 grid(x.a.B * x.cfg.hkv * x.a.lq);
  if (x.cfg.d == 128) launch_combine_d<128>(x, grid, st);
  else launch_combine_d<64>(x, grid, st);
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
  if (a.lq >= kPrefillMinLq) {
    launch_prefill(x, st);
    launch_combine(x, st);
    return hipGetLastError();
  }
  dim3 grid(x.n_splits, cfg.hkv, a.B * a.lq);
  if (cfg.d == 128) launch_d<128>(x, grid, st);
  else launch_d<64>(x, grid, st);
  return hipGetLastError();
}

}  // namespace hga
