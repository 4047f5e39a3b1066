// Two-level chunk -> group routing with the deterministic visibility windows.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 2: the current
// query scores a compact table of chunk key summaries (level 1), then the
// group key summaries inside the chosen chunks (level 2); the current chunk,
// the first sink chunks and the most recent local chunks are always visible.
//
// Two launches per call.
//  route_tiles: grid = (tiles of 64 candidate chunks, Hkv, B), 256 threads.
//    Each workgroup forms the pooled routing query qbar (mean over the KV
//    head's query heads and query tokens of RoPE(q, position), fp64) and
//    scores its tile: a 512-byte summary row is read by 8 lanes (4 x 16 B
//    each, one wave instruction covering 8 rows), fp64 dot, fp64 DPP sum over
//    the 8 lanes, fp64 score to the workspace.  Tile 0 also stores qbar.
//  route_select: one workgroup per (sequence, KV head).  Level-1 top-k over
//    the scores, level-2 scores of the G groups of every kept chunk (all row
//    loads in flight at once), level-2 top-k, and the ascending group list.
//    The kernel boundary makes the first launch's scores visible to the
//    second with plain loads.
// Top-k (the whole workgroup for up to 1024 scores, one wave streaming from
// LDS beyond): a 256-bin histogram between the min and max score finds the
// bin holding the k-th largest score; every score in a higher bin is kept,
// and the boundary bin is resolved exactly by rank counting with the order
// (score descending, id ascending).  Scores stay
// fp64 throughout, so the kept set equals the fp64 reference wherever its
// score gap exceeds the error of the fp32-stored summaries.
#include "hga_build_dev.h"
#include "hga_topk.h"

namespace hga {

constexpr int kTile = 64;       // candidate chunks per tile workgroup
constexpr int kLanesPerRow = 8; // lanes per summary row

struct RouteArgs {
  KCfg cfg;
  RouteLaunch r;
  int max_cand;
  StepFront f;  // used by the workgroups with blockIdx.z == 1 of route_select
};

// Position and candidate range of a unit; false if the query position is
// unusable (negative, query tokens spanning two chunks, a query chunk beyond
// the summary table, or, in a fused step, tokens beyond the pool).
__device__ __forceinline__ bool route_geometry(const KCfg& c, const RouteLaunch& r, int max_cand,
                                               int b, int* pos0, Windows* w) {
  *pos0 = r.q_pos0[b];
  *w = windows_of(*pos0 / kChunk, c.n_sink, c.n_local);
  return *pos0 >= 0 && (*pos0 % kChunk) + r.lq <= kChunk && *pos0 / kChunk < r.max_chunks &&
         w->cand_hi - w->cand_lo <= max_cand && (r.pool_cap <= 0 || *pos0 + r.lq <= r.pool_cap);
}

// MODE 0: pooled query of up to S tokens + scores (decode);
// MODE 1: pooled query of more tokens (chunked prefill) + scores, a separate
//         instantiation so that the decode form keeps its small register
//         footprint;
// MODE 2: the multi-token pooled query only (grid x = 1), stored for MODE 3;
// MODE 3: scores only, with the stored pooled query.  The whole-prompt
//         prefill runs 2 then 3, so the query of a chunk is pooled once
//         instead of once per tile.
template <int D, bool BF16, int MODE>
__global__ __launch_bounds__(256) void route_tiles_kernel(RouteArgs a) {
  constexpr int P = D / 2;
  constexpr int S = 256 / P;                 // query-token slices
  constexpr int NV = D / 32;                 // float4 per lane per row
  constexpr int RPI = 64 / kLanesPerRow;     // rows per wave instruction
  constexpr int ITER = (kTile / 4) / RPI;    // row passes per wave
  using T = typename std::conditional<BF16, uint16_t, float>::type;

  constexpr int JP = P / 2;                  // multi-token path: two adjacent pairs per thread
  constexpr int S2 = 256 / JP;               // multi-token path: query-token slices
  constexpr int TPT = kChunk / S2;           // multi-token path: tokens per thread (max)
  using QT = typename std::conditional<BF16, uint32_t, float2>::type;  // two adjacent dims
  constexpr int TB = BF16 ? 4 : 2;           // multi-token path: tokens per load batch (64 VGPRs)
  static_assert(TPT % TB == 0, "token batches");
  __shared__ double qpart[S2][P][2];
  __shared__ double qbar[D];

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int unit = b * c.lists + h;                  // workspace rows: virtual sequence, list
  const int unit_p = (b / r.nq) * c.hkv + h / c.kvdiv;  // summaries: pool sequence, KV head
  const size_t qhead0 = (size_t)(b / r.nq) * c.hq + (size_t)h * c.lhg;
  const int qt0 = (b % r.nq) * r.lq;              // first query row of this chunk
  const int lq = r.lq;
  int pos0;
  Windows w;
  if (!route_geometry(c, r, a.max_cand, b, &pos0, &w)) return;  // route_select reports it
  const int n_cand = w.cand_hi - w.cand_lo;
  const int tile0 = blockIdx.x * kTile;
  constexpr bool multi = MODE == 1 || MODE == 2;
  constexpr bool pool_q = MODE != 3;    // this launch forms the pooled query
  constexpr bool score = MODE != 2;     // this launch scores its tile
  if (tile0 >= n_cand && (blockIdx.x != 0 || !pool_q)) return;  // tile 0 stores qbar

  // ---- loads: the query first, then the tile's summary rows.  Rows past
  // the candidates are read from a clamped in-range row (so every load
  // issues together) and ignored.
  //   up to S query tokens: thread (j, sl) loads pair j of every query head
  //   of this KV head for token sl;
  //   more tokens (prefill): thread (jp, sl2) loads pairs 2jp, 2jp + 1 (two
  //   adjacent dims of each half) for tokens sl2, sl2 + S2, ..., in batches
  //   of TB tokens with all their loads in flight (clamped to the last
  //   token; extras ignored).
  const int j = tid % P, sl = tid / P;
  const int jp = tid % JP, sl2 = tid / JP;
  const T* q = static_cast<const T*>(r.q);
  T xa[8], xb[8];
  QT ya[TB][8], yb[TB][8];
  // dims of the two 2-element loads of pairs 2jp, 2jp + 1: half-split (a of
  // both, b of both) or interleaved (a, b of pair 2jp; a, b of pair 2jp + 1)
  const int qoa = c.interleaved ? 4 * jp : 2 * jp;
  const int qob = c.interleaved ? 4 * jp + 2 : P + 2 * jp;
  auto load_batch = [&](int u0) {  // tokens sl2 + (u0 + u) * S2, u < TB
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int tt = sl2 + (u0 + u) * S2;
      const int t = tt < lq ? tt : lq - 1;
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) {
        const int hc = hh < c.lhg ? hh : c.lhg - 1;
        const size_t row = ((qhead0 + hc) * r.q_tokens + qt0 + t) * D;
        ya[u][hh] = *reinterpret_cast<const QT*>(q + row + qoa);
        yb[u][hh] = *reinterpret_cast<const QT*>(q + row + qob);
      }
    }
  };
  if constexpr (!pool_q) {
  } else if constexpr (!multi) {
    const int t0 = sl < lq ? sl : lq - 1;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      const int hc = hh < c.lhg ? hh : c.lhg - 1;
      const size_t row = ((qhead0 + hc) * r.q_tokens + qt0 + t0) * D;
      xa[hh] = q[row + pair_a(c, j)];
      xb[hh] = q[row + pair_b(c, j)];
    }
  } else {
    load_batch(0);
  }
  const int sub = lane % kLanesPerRow, rin = lane / kLanesPerRow;
  float4 buf[ITER][NV];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    if constexpr (!score) break;
    int idx = tile0 + wave * (kTile / 4) + it * RPI + rin;
    idx = idx < n_cand ? w.cand_lo + idx : (n_cand > 0 ? w.cand_hi - 1 : 0);
    const float4* rowp =
        reinterpret_cast<const float4*>(r.chunk_sum + ((size_t)unit_p * r.max_chunks + idx) * D);
#pragma unroll
    for (int v = 0; v < NV; ++v) buf[it][v] = rowp[v * kLanesPerRow + sub];
  }

  // ---- pooled routing query (fp64): the query heads of this KV head are
  // summed per token and dim, the head sum of each token is rotated to the
  // token's position once, and the rotated sums are added over tokens.  The
  // angle of a thread's next token follows by one fp64 rotation by the
  // token stride times omega_j (error ~1e-16 per step).
  if constexpr (pool_q) {
    auto to_d = [](T x) -> double {
      if constexpr (BF16) return bf16_to_f(x);
      else return x;
    };
    if constexpr (!multi) {
      if (sl < lq) {
        double x = 0.0, y = 0.0;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh)
          if (hh < c.lhg) {
            x += to_d(xa[hh]);
            y += to_d(xb[hh]);
          }
        double cs, sn;
        rope_cs((double)(pos0 + sl), c.omega[j], &cs, &sn);
        qpart[sl][j][0] = x * cs - y * sn;
        qpart[sl][j][1] = x * sn + y * cs;
      } else {
        qpart[sl][j][0] = 0.0;
        qpart[sl][j][1] = 0.0;
      }
    } else {
      double qa[2] = {0.0, 0.0}, qb[2] = {0.0, 0.0};
      double cs[2], sn[2], cd[2], sd[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const double wj = c.omega[2 * jp + e];
        rope_cs((double)(pos0 + sl2), wj, &cs[e], &sn[e]);
        sincos((double)S2 * wj, &sd[e], &cd[e]);
      }
      for (int u0 = 0; u0 < TPT && sl2 + u0 * S2 < lq; u0 += TB) {
        if (u0 > 0) load_batch(u0);
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          if (sl2 + (u0 + u) * S2 < lq) {
            double x[2] = {0.0, 0.0}, y[2] = {0.0, 0.0};
#pragma unroll
            for (int hh = 0; hh < 8; ++hh)
              if (hh < c.lhg) {
                double e0, e1, e2, e3;  // the four loaded elements in load order
                if constexpr (BF16) {
                  e0 = bf16_to_f((uint16_t)(ya[u][hh] & 0xFFFFu));
                  e1 = bf16_to_f((uint16_t)(ya[u][hh] >> 16));
                  e2 = bf16_to_f((uint16_t)(yb[u][hh] & 0xFFFFu));
                  e3 = bf16_to_f((uint16_t)(yb[u][hh] >> 16));
                } else {
                  e0 = ya[u][hh].x;
                  e1 = ya[u][hh].y;
                  e2 = yb[u][hh].x;
                  e3 = yb[u][hh].y;
                }
                x[0] += e0;
                x[1] += c.interleaved ? e2 : e1;
                y[0] += c.interleaved ? e1 : e2;
                y[1] += e3;
              }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              qa[e] += x[e] * cs[e] - y[e] * sn[e];
              qb[e] += x[e] * sn[e] + y[e] * cs[e];
            }
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const double c2 = cs[e] * cd[e] - sn[e] * sd[e];
            sn[e] = sn[e] * cd[e] + cs[e] * sd[e];
            cs[e] = c2;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        qpart[sl2][2 * jp + e][0] = qa[e];
        qpart[sl2][2 * jp + e][1] = qb[e];
      }
    }
    __syncthreads();
    if (tid < P) {
      const int ns = multi ? S2 : S;
      double sa = 0.0, sb = 0.0;
      for (int u = 0; u < ns; ++u) {
        sa += qpart[u][tid][0];
        sb += qpart[u][tid][1];
      }
      const double inv = 1.0 / (double)(c.lhg * lq);
      qbar[pair_a(c, tid)] = sa * inv;
      qbar[pair_b(c, tid)] = sb * inv;
      if (blockIdx.x == 0) {
        r.qbar[(size_t)unit * D + pair_a(c, tid)] = sa * inv;
        r.qbar[(size_t)unit * D + pair_b(c, tid)] = sb * inv;
      }
    }
    __syncthreads();
  }
  if constexpr (!score) return;

  // ---- level-1 scores of this tile
#pragma unroll
  for (int it = 0; it < ITER; ++it)
#pragma unroll
    for (int v = 0; v < NV; ++v) hold(buf[it][v]);
  double qv[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * (v * kLanesPerRow + sub) + e;
      qv[v][e] = pool_q ? qbar[i] : r.qbar[(size_t)unit * D + i];
    }
  double* scores = r.scores + (size_t)unit * a.max_cand;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = tile0 + wave * (kTile / 4) + it * RPI + rin;
    double d = 0.0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      d = fma((double)buf[it][v].x, qv[v][0], d);
      d = fma((double)buf[it][v].y, qv[v][1], d);
      d = fma((double)buf[it][v].z, qv[v][2], d);
      d = fma((double)buf[it][v].w, qv[v][3], d);
    }
    d = group8_sum_d(d);
    if (sub == 0 && idx < n_cand) {
      const double sc = d * c.inv_sqrt_d;
      scores[idx] = sc;
      if (r.chunk_scores) r.chunk_scores[(size_t)unit * r.max_chunks + w.cand_lo + idx] = sc;
    }
  }
}

// Token work of a fused step for unit (h, b), on one workgroup: the raw
// keys of the step's lq tokens go to their staging rows, their rotated keys
// and values to the pool (the same arithmetic as hga_build_summaries over
// those tokens), and when the last token ends its chunk the chunk's
// summaries are built from the staging rows of the earlier positions plus
// the new keys.  Neither is read by this step's routing: the current chunk
// is never a candidate.  An unusable position (as route_geometry) writes
// nothing.
template <int D, bool BF16>
__device__ void step_front(const RouteArgs& a, int h, int b, double* lds) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  const KCfg& c = a.cfg;
  const StepFront& f = a.f;
  const int unit = b * c.hkv + h;
  const int pos = a.r.q_pos0[b];
  const int lq = a.r.lq;
  if (pos < 0 || (pos % kChunk) + lq > kChunk || pos / kChunk >= a.r.max_chunks ||
      pos + lq > f.pool_cap)
    return;  // route_select reports the position
  const int c0 = pos / kChunk * kChunk;
  const T* kn = static_cast<const T*>(f.k_new) + (size_t)unit * lq * D;
  const T* vn = static_cast<const T*>(f.v_new) + (size_t)unit * lq * D;
  T* stage = static_cast<T*>(f.k_stage) + (size_t)unit * kChunk * D;
  // a plain pool, or the FP8 pool (codes and row scales of each of the step's
  // tokens, appended one row at a time by a small routine of its own)
  T* kp = c.pool8 ? nullptr : static_cast<T*>(f.k_pool) + (size_t)unit * f.pool_cap * D;
  T* vp = c.pool8 ? nullptr : static_cast<T*>(f.v_pool) + (size_t)unit * f.pool_cap * D;
  if constexpr (D == 128 && BF16) {
    if (c.pool8) {  // lq <= 15 (checked on the host)
      const Fp8Rows f8 = fp8_rows_of(f.k_pool, f.v_pool, a.r.B * c.hkv, f.pool_cap, D, unit);
      for (int p = pos; p < pos + lq; ++p)
        fp8_append_row(c, static_cast<const uint16_t*>(f.k_new) + ((size_t)unit * lq + (p - pos)) * D,
                       static_cast<const uint16_t*>(f.v_new) + ((size_t)unit * lq + (p - pos)) * D,
                       c0, p, f8);
    }
  }
  auto knew = [&](int p) { return kn + (size_t)(p - pos) * D; };
  auto vnew = [&](int p) { return vn + (size_t)(p - pos) * D; };
  const int chunk = pos / kChunk;
  float* cs = f.chunk_sum + ((size_t)unit * a.r.max_chunks + chunk) * D;
  float* gs = f.group_sum + ((size_t)unit * a.r.max_chunks + chunk) * kGroups * D;
  const bool ends = pos + lq - c0 == kChunk;  // uniform
  if (ends && pos == c0) {  // the whole chunk in this step: one pass
    build_span<D, BF16>(c, c0, pos, pos + lq, knew, vnew, kp, vp, cs, gs, lds, stage);
    return;
  }
  build_span<D, BF16>(c, c0, pos, pos + lq, knew, vnew, kp, vp, nullptr, nullptr, lds, stage);
  if (ends) {
    build_span<D, BF16>(
        c, c0, c0, c0 + kChunk,
        [&](int p) { return p >= pos ? knew(p) : stage + (size_t)(p - c0) * D; },
        [&](int) { return kn; }, static_cast<T*>(nullptr), static_cast<T*>(nullptr), cs, gs, lds);
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a) {
  constexpr int NV = D / 32;
  constexpr int RPP = 256 / kLanesPerRow;  // rows per pass of the workgroup
  constexpr int U = 8;                     // passes in flight
  __shared__ int hist[256];
  __shared__ int kk[2];
  __shared__ double red[8];
  __shared__ int ints[8];
  extern __shared__ double dyn[];

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  if (blockIdx.z == 1) {  // a fused step's token work, once per KV head
    if (h % c.kvdiv == 0) step_front<D, BF16>(a, h / c.kvdiv, b, dyn);
    return;
  }
  const int unit = b * c.lists + h;                     // lists and workspace: virtual sequence
  const int unit_p = (b / r.nq) * c.hkv + h / c.kvdiv;  // summaries: pool sequence, KV head

  // every load that does not depend on the position goes out first: this
  // lane's qbar slice (for level 2) and the level-1 scores (clamped to the
  // table; entries past the candidates are dropped below)
  const int sub = lane % kLanesPerRow;
  double qv[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      qv[v][e] = r.qbar[(size_t)unit * D + 4 * (v * kLanesPerRow + sub) + e];
  const double* scores = r.scores + (size_t)unit * a.max_cand;
  constexpr int SPT = 4;  // scores per thread in flight
  double v4[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int i = u * 256 + tid;
    v4[u] = scores[i < a.max_cand ? i : a.max_cand - 1];
  }

  int pos0;
  Windows w;
  if (!route_geometry(c, r, a.max_cand, b, &pos0, &w)) {
    if (tid == 0) r.n_sel[unit] = -1;
    return;
  }
  const int n_cand = w.cand_hi - w.cand_lo;
  const int ct = pos0 / kChunk;

  const int n2max = c.topk_c * kGroups;
  const int nmax = a.max_cand > n2max ? a.max_cand : n2max;
  // LDS: scores | boundary list | boundary winners | level-1 list | level-2 list
  double* s_lds = dyn;
  int* bl = reinterpret_cast<int*>(s_lds + nmax);
  int* win = bl + nmax;
  int* sel = win + nmax;
  int* sel2 = sel + nmax;
  const TopkScratch tks{hist, bl, win};
  const BlockTopkScratch bts{hist, bl, red, ints};

  double mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int i = u * 256 + tid;
    if (i < n_cand) {
      s_lds[i] = v4[u];
      mn1 = fmin(mn1, v4[u]);
      mx1 = fmax(mx1, v4[u]);
    }
  }
  for (int i = SPT * 256 + tid; i < n_cand; i += 256) s_lds[i] = scores[i];
  topk_publish(mn1, mx1, bts);
  __syncthreads();
  // level 1: kept candidate indices, ascending, into sel
  int k1;
  if (n_cand <= 1024) {
    k1 = block_topk(s_lds, n_cand, c.topk_c, sel, bts);
  } else {  // long candidate lists: one wave streams them from LDS
    if (wave == 0) {
      const int k = wave_topk(s_lds, n_cand, c.topk_c, sel, tks);
      if (lane == 0) kk[0] = k;
    }
    __syncthreads();
    k1 = kk[0];
  }

  // level 2 (all waves): the G groups of each kept chunk
  const int n2 = k1 * kGroups;
  const int rsub = tid / kLanesPerRow;
  double mn2 = INFINITY, mx2 = -INFINITY;
  for (int base = 0; base < n2; base += RPP * U) {
    float4 gb[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int i = base + u * RPP + rsub;
      i = i < n2 ? i : n2 - 1;  // clamped: every load issues, extras ignored
      const int gid = (w.cand_lo + sel[i / kGroups]) * kGroups + i % kGroups;
      const float4* rowp = reinterpret_cast<const float4*>(
          r.group_sum + ((size_t)unit_p * r.max_chunks * kGroups + gid) * D);
#pragma unroll
      for (int v = 0; v < NV; ++v) gb[u][v] = rowp[v * kLanesPerRow + sub];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * RPP + rsub;
      double d = 0.0;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        d = fma((double)gb[u][v].x, qv[v][0], d);
        d = fma((double)gb[u][v].y, qv[v][1], d);
        d = fma((double)gb[u][v].z, qv[v][2], d);
        d = fma((double)gb[u][v].w, qv[v][3], d);
      }
      d = group8_sum_d(d) * c.inv_sqrt_d;
      if (sub == 0 && i < n2) {
        s_lds[i] = d;
        mn2 = fmin(mn2, d);
        mx2 = fmax(mx2, d);
      }
    }
  }
  topk_publish(mn2, mx2, bts);
  __syncthreads();
  // level 2 selection: kept group indices, ascending = gid order
  int k2;
  if (n2 <= 1024) {
    k2 = block_topk(s_lds, n2, c.topk_g, sel2, bts);
  } else {
    if (wave == 0) {
      const int k = wave_topk(s_lds, n2, c.topk_g, sel2, tks);
      if (lane == 0) kk[1] = k;
    }
    __syncthreads();
    k2 = kk[1];
  }

  // the list: sink | routed | local | current
  const int last = pos0 + r.lq - 1;
  const int n_head = w.sink_end * kGroups;
  const int n_local = (ct - w.local_begin) * kGroups;
  const int n_cur = last / kGroupTokens - ct * kGroups + 1;
  const int n_sel = n_head + k2 + n_local + n_cur;
  int* out = r.sel + (size_t)unit * r.max_sel;
  for (int i = tid; i < n_sel; i += 256) {
    int gid;
    if (i < n_head) {
      gid = i;
    } else if (i < n_head + k2) {
      const int x = sel2[i - n_head];
      gid = (w.cand_lo + sel[x / kGroups]) * kGroups + x % kGroups;
    } else {
      gid = w.local_begin * kGroups + (i - n_head - k2);
    }
    out[i] = gid;
  }
  if (tid == 0) r.n_sel[unit] = n_sel;
}

static int max_cand_of(const KCfg& cfg, int max_chunks) {
  return max_chunks > cfg.n_sink ? max_chunks - cfg.n_sink : 1;
}

size_t route_ws_bytes(const KCfg& cfg, int B, int max_chunks) {
  return (size_t)B * cfg.lists * (max_cand_of(cfg, max_chunks) + cfg.d) * sizeof(double);
}

size_t route_select_lds(const KCfg& cfg, int max_chunks) {
  const int max_cand = max_cand_of(cfg, max_chunks);
  const int n2 = cfg.topk_c * kGroups;
  const size_t nmax = (size_t)(max_cand > n2 ? max_cand : n2);
  return nmax * (sizeof(double) + 3 * sizeof(int)) + (size_t)n2 * sizeof(int);
}

template <int D, bool BF16>
static void launch_tiles(bool multi, bool pooled_once, dim3 grid, hipStream_t st,
                         const RouteArgs& a) {
  if (pooled_once) {  // pooled query once per unit, then the tiles
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 2>), dim3(1, grid.y, grid.z), dim3(256), 0, st, a);
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 3>), grid, dim3(256), 0, st, a);
  } else if (multi) {
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 1>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 0>), grid, dim3(256), 0, st, a);
  }
}

hipError_t launch_route(const KCfg& cfg, const RouteLaunch& r, hipStream_t st,
                        const StepFront* front) {
  RouteArgs a{};
  a.cfg = cfg;
  a.r = r;
  a.max_cand = max_cand_of(cfg, r.max_chunks);
  if (front) a.f = *front;
  const int n_tiles = (a.max_cand + kTile - 1) / kTile;
  size_t lds = route_select_lds(cfg, r.max_chunks);
  const size_t front_lds = (size_t)256 * 2 * sizeof(double);  // build_span scratch: S*P*2 doubles
  if (front && lds < front_lds) lds = front_lds;
  dim3 grid(n_tiles, cfg.lists, r.B);
  dim3 sgrid(cfg.lists, r.B, front ? 2 : 1);
  const bool bf = cfg.dtype == HGA_BF16;
  const bool multi = r.lq > 256 / (cfg.d / 2);  // more tokens than slices
  if (cfg.d == 128) {
    if (bf) {
      launch_tiles<128, true>(multi, r.pool_once, grid, st, a);
      hipLaunchKernelGGL((route_select_kernel<128, true>), sgrid, dim3(256), lds, st, a);
    } else {
      launch_tiles<128, false>(multi, r.pool_once, grid, st, a);
      hipLaunchKernelGGL((route_select_kernel<128, false>), sgrid, dim3(256), lds, st, a);
    }
  } else {
    if (bf) {
      launch_tiles<64, true>(multi, r.pool_once, grid, st, a);
      hipLaunchKernelGGL((route_select_kernel<64, true>), sgrid, dim3(256), lds, st, a);
    } else {
      launch_tiles<64, false>(multi, r.pool_once, grid, st, a);
      hipLaunchKernelGGL((route_select_kernel<64, false>), sgrid, dim3(256), lds, st, a);
    }
  }
  return hipGetLastError();
}

}  // namespace hga
