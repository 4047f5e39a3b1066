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
//    the scores, level-2 scores of the G groups of every kept chunk, level-2
//    top-k, and the ascending group list.  The kernel boundary makes the
//    first launch's scores visible to the second with plain loads.
// The tile workgroups issue their query and summary-row loads before the
// position arrives, and also store the score range of every 16 rows, so the
// selection can bin its scores without a reduction of its own.
// Selection (route_select_fast_kernel, up to 1024 candidates and 64 kept
// chunks): histogram selection with member slots (hga_topk.h) at both
// levels; between them one barrier publishes every wave's kept chunks and the
// group rows of all kept chunks are dealt evenly over the four waves.  Longer candidate
// lists run route_select_kernel: a 256-bin histogram between the min and max
// score finds the bin holding the k-th largest score, every score in a
// higher bin is kept, and the boundary bin is resolved exactly by rank
// counting with the order (score descending, id ascending).  Scores stay fp64
// throughout, so the kept set equals the fp64 reference wherever its score
// gap exceeds the error of the fp32-stored summaries.
#include "hga_build_dev.h"
#include "hga_topk.h"

namespace hga {

// A 16-byte summary-row load that is read once per step: non-temporal, so
// that the streamed rows do not displace cached lines (the scores, lists
// and code the next kernels of the step read)
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_row_nt(const float4* p) {
  const f32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

constexpr int kTile = 64;       // candidate chunks per tile workgroup
constexpr int kLanesPerRow = 8; // lanes per summary row
constexpr int kMaxHg = 8;       // query heads per list (max pooling keeps one query each)

// Max pooling: the largest over the nh routing queries q [nh][D] (fp64, LDS)
// of their dot products with a summary row held by 8 lanes (NV float4 per
// lane, this lane's sub-slice sub), before the 1/sqrt(d) factor.
template <int NV>
__device__ __forceinline__ double route_row_max(const float4 (&row)[NV], const double* q, int nh,
                                                int sub) {
  constexpr int D = NV * 32;
  double best = -INFINITY;
  for (int hh = 0; hh < nh; ++hh) {
    const double* qq = q + (size_t)hh * D;
    double d = 0.0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int i = 4 * (v * kLanesPerRow + sub);
      d = fma((double)row[v].x, qq[i], d);
      d = fma((double)row[v].y, qq[i + 1], d);
      d = fma((double)row[v].z, qq[i + 2], d);
      d = fma((double)row[v].w, qq[i + 3], d);
    }
    best = fmax(best, group8_sum_d(d));
  }
  return best;
}

struct RouteArgs {
  KCfg cfg;
  RouteLaunch r;
  int max_cand;
  int score_ld;     // workspace row stride of the level-1 scores (max_cand rounded up to 4)
  int n_tiles;      // tile workgroups per unit
  double* ranges;   // workspace [units][n_tiles * 4] of (min, max): the level-1 scores of
                    // rows 16 l .. 16 l + 15 of the candidates (wave l % 4 of tile l / 4)
  StepFront f;      // used by the workgroups with blockIdx.z >= 1 of route_select
};

// Position and candidate range of a unit; false if the query position is
// unusable (negative, query tokens spanning two chunks, a query chunk beyond
// the summary table, or, in a fused step, tokens beyond the pool).
__device__ __forceinline__ bool route_geometry_at(const KCfg& c, const RouteLaunch& r,
                                                  int max_cand, int p0, int* pos0, Windows* w) {
  *pos0 = p0;
  *w = windows_of(*pos0 / kChunk, c.n_sink, c.n_local);
  return *pos0 >= 0 && (*pos0 % kChunk) + r.lq <= kChunk && *pos0 / kChunk < r.max_chunks &&
         w->cand_hi - w->cand_lo <= max_cand && (r.pool_cap <= 0 || *pos0 + r.lq <= r.pool_cap);
}
__device__ __forceinline__ bool route_geometry(const KCfg& c, const RouteLaunch& r, int max_cand,
                                               int b, int* pos0, Windows* w) {
  return route_geometry_at(c, r, max_cand, r.q_pos0[b], pos0, w);
}

// MODE 0: pooled query of up to S tokens + scores (decode);
// MODE 1: pooled query of more tokens (chunked prefill) + scores, a separate
//         instantiation so that the decode form keeps its small register
//         footprint;
// MODE 2: the multi-token pooled query only (grid x = 1), stored for MODE 3;
// MODE 3: scores only, with the stored pooled query.  The whole-prompt
//         prefill runs 2 then 3, so the query of a chunk is pooled once
//         instead of once per tile.
template <int D, bool BF16, int MODE, bool MAXQ = false>
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
  // multi-token path: tokens per load batch (bf16: every token of the thread at once)
  constexpr int TB = BF16 ? TPT : 2;
  static_assert(TPT % TB == 0, "token batches");
  __shared__ double qpart[S2][P][2];
  __shared__ double qbar[D];
  __shared__ double qh[MAXQ ? kMaxHg : 1][D];  // max pooling: each query head's routing query

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int unit = b * c.lists + h;                  // workspace rows: virtual sequence, list
  const int unit_p = (b / r.nq) * c.hkv + h / c.kvdiv;  // summaries: pool sequence, KV head
  const size_t qhead0 = (size_t)(b / r.nq) * c.hq + (size_t)h * c.lhg;
  const int qt0 = (b % r.nq) * r.lq;              // first query row of this chunk
  const int lq = r.lq;
  const int tile0 = blockIdx.x * kTile;
  const int pos0_in = r.q_pos0[b];  // first: a scalar load ahead of everything
  constexpr bool multi = MODE == 1 || MODE == 2;
  constexpr bool pool_q = MODE != 3;    // this launch forms the pooled query
  constexpr bool score = MODE != 2;     // this launch scores its tile

  // ---- loads, issued before the position arrives: the query first, then
  // the tile's summary rows (candidates start at chunk n_sink whatever the
  // position).  Rows past the table are read from a clamped in-range row
  // (so every load issues together) and ignored.
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
  // this thread's RoPE frequencies (kernel arguments indexed by lane: a
  // vector load, issued here so that it is not queued behind the row loads)
  double om[2] = {0.0, 0.0};
  if constexpr (pool_q && !multi) {
    om[0] = c.omega[j];
  } else if constexpr (pool_q) {
    om[0] = c.omega[2 * jp];
    om[1] = c.omega[2 * jp + 1];
  }
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
  // the query loads go out ahead of the row loads (the rows are the bulk of
  // the traffic; a query load queued behind them delays the pooled query)
  __builtin_amdgcn_sched_barrier(0);
  const int sub = lane % kLanesPerRow, rin = lane / kLanesPerRow;
  float4 buf[ITER][NV];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    if constexpr (!score) break;
    int row = c.n_sink + tile0 + wave * (kTile / 4) + it * RPI + rin;
    row = row < r.max_chunks ? row : r.max_chunks - 1;
    const float4* rowp =
        reinterpret_cast<const float4*>(r.chunk_sum + ((size_t)unit_p * r.max_chunks + row) * D);
#pragma unroll
    for (int v = 0; v < NV; ++v) buf[it][v] = load_row_nt(rowp + v * kLanesPerRow + sub);
  }

  // ... and stay ahead of the exits below (the compiler would otherwise sink
  // them past the exits, behind every row load): this waits for the query
  // values only, the row loads issued after them stay in flight
  if constexpr (pool_q && !multi) {
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) asm volatile("" ::"v"(xa[hh]), "v"(xb[hh]));
    asm volatile("" ::"v"(om[0]));
  } else if constexpr (pool_q) {
    asm volatile("" ::"v"(om[0]), "v"(om[1]));
#pragma unroll
    for (int u = 0; u < TB; ++u)
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) asm volatile("" ::"v"(ya[u][hh]), "v"(yb[u][hh]));
  }
  int pos0;
  Windows w;
  if (!route_geometry_at(c, r, a.max_cand, pos0_in, &pos0, &w)) return;  // route_select reports it
  const int n_cand = w.cand_hi - w.cand_lo;
  if (tile0 >= n_cand && (blockIdx.x != 0 || !pool_q)) return;  // tile 0 stores qbar

  // ---- pooled routing query (fp64): the query heads of this KV head are
  // summed per token and dim, the head sum of each token is rotated to the
  // token's position once, and the rotated sums are added over tokens.  The
  // angle of a thread's next token follows by one fp64 rotation by the
  // token stride times omega_j (error ~1e-16 per step).
  // Max pooling: the same per query head (no sum over the heads), one head
  // at a time through qpart; qh[h] = head h's mean over the query tokens.
  auto reduce_head = [&](int hh) {
    if (tid < P) {
      const int ns = multi ? S2 : S;
      double sa = 0.0, sb = 0.0;
      for (int u = 0; u < ns; ++u) {
        sa += qpart[u][tid][0];
        sb += qpart[u][tid][1];
      }
      const double inv = 1.0 / (double)lq;
      qh[hh][pair_a(c, tid)] = sa * inv;
      qh[hh][pair_b(c, tid)] = sb * inv;
      if (blockIdx.x == 0) {
        r.qbar[((size_t)unit * c.lhg + hh) * D + pair_a(c, tid)] = sa * inv;
        r.qbar[((size_t)unit * c.lhg + hh) * D + pair_b(c, tid)] = sb * inv;
      }
    }
  };
  if constexpr (pool_q && MAXQ) {
    auto to_d = [](T x) -> double {
      if constexpr (BF16) return bf16_to_f(x);
      else return x;
    };
    if constexpr (!multi) {
      double cs = 1.0, sn = 0.0;
      if (sl < lq) rope_cs((double)(pos0 + sl), om[0], &cs, &sn);
#pragma unroll
      for (int hh = 0; hh < kMaxHg; ++hh) {
        if (hh >= c.lhg) break;  // uniform
        const double x = sl < lq ? to_d(xa[hh]) : 0.0, y = sl < lq ? to_d(xb[hh]) : 0.0;
        qpart[sl][j][0] = x * cs - y * sn;
        qpart[sl][j][1] = x * sn + y * cs;
        __syncthreads();
        reduce_head(hh);
        __syncthreads();
      }
    } else {
      double qa[kMaxHg][2], qb[kMaxHg][2];
#pragma unroll
      for (int hh = 0; hh < kMaxHg; ++hh) qa[hh][0] = qa[hh][1] = qb[hh][0] = qb[hh][1] = 0.0;
      double cs[2], sn[2], cd[2], sd[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const double wj = om[e];
        rope_cs((double)(pos0 + sl2), wj, &cs[e], &sn[e]);
        sincos_rad((double)S2 * wj, &sd[e], &cd[e]);
      }
      for (int u0 = 0; u0 < TPT && sl2 + u0 * S2 < lq; u0 += TB) {
        if (u0 > 0) load_batch(u0);
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          if (sl2 + (u0 + u) * S2 < lq) {
#pragma unroll
            for (int hh = 0; hh < kMaxHg; ++hh)
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
                const double x[2] = {e0, c.interleaved ? e2 : e1};
                const double y[2] = {c.interleaved ? e1 : e2, e3};
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                  qa[hh][e] += x[e] * cs[e] - y[e] * sn[e];
                  qb[hh][e] += x[e] * sn[e] + y[e] * cs[e];
                }
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
      for (int hh = 0; hh < kMaxHg; ++hh) {
        if (hh >= c.lhg) break;  // uniform
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          qpart[sl2][2 * jp + e][0] = qa[hh][e];
          qpart[sl2][2 * jp + e][1] = qb[hh][e];
        }
        __syncthreads();
        reduce_head(hh);
        __syncthreads();
      }
    }
  } else if constexpr (pool_q) {
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
        rope_cs((double)(pos0 + sl), om[0], &cs, &sn);
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
        const double wj = om[e];
        rope_cs((double)(pos0 + sl2), wj, &cs[e], &sn[e]);
        sincos_rad((double)S2 * wj, &sd[e], &cd[e]);
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
  if constexpr (MAXQ && !pool_q) {  // the stored per-head routing queries
    for (int i = tid; i < c.lhg * D; i += 256) qh[i / D][i % D] = r.qbar[(size_t)unit * c.lhg * D + i];
    __syncthreads();
  }
  double qv[NV][4];
  if constexpr (!MAXQ) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * (v * kLanesPerRow + sub) + e;
        qv[v][e] = pool_q ? qbar[i] : r.qbar[(size_t)unit * D + i];
      }
  }
  double* scores = r.scores + (size_t)unit * a.score_ld;
  double rmn = INFINITY, rmx = -INFINITY;  // this wave's score range (its 16 rows)
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = tile0 + wave * (kTile / 4) + it * RPI + rin;
    double d = 0.0;
    if constexpr (MAXQ) {
      d = route_row_max<NV>(buf[it], &qh[0][0], c.lhg, sub);
    } else {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        d = fma((double)buf[it][v].x, qv[v][0], d);
        d = fma((double)buf[it][v].y, qv[v][1], d);
        d = fma((double)buf[it][v].z, qv[v][2], d);
        d = fma((double)buf[it][v].w, qv[v][3], d);
      }
      d = group8_sum_d(d);
    }
    if (sub == 0 && idx < n_cand) {
      const double sc = d * c.inv_sqrt_d;
      scores[idx] = sc;
      rmn = fmin(rmn, sc);
      rmx = fmax(rmx, sc);
      if (r.chunk_scores) r.chunk_scores[(size_t)unit * r.max_chunks + w.cand_lo + idx] = sc;
    }
  }
  rmn = wave_ext_d<false>(rmn);
  rmx = wave_ext_d<true>(rmx);
  if (lane == 0)
    reinterpret_cast<double2*>(a.ranges)[(size_t)unit * a.n_tiles * 4 + blockIdx.x * 4 + wave] =
        make_double2(rmn, rmx);
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

// The token work of a step of many tokens spread over kFrontParts
// workgroups per unit: part 0 builds the chunk's summaries (no row stores),
// part 1 + g appends the step's tokens of group g of the chunk (rows and
// staging rows, no summaries).  Every row and sum is computed as step_front
// computes it (build_span steps the angles of a 16-token group from the
// group's first position either way), so the results are the same bits;
// what is spread is the row stores, which one workgroup would issue through
// a single CU.
constexpr int kFrontParts = 1 + kGroups;
constexpr int kFrontSplitLq = kGroupTokens;  // steps of at least a group of tokens split their work

template <int D, bool BF16>
__device__ void step_front_part(const RouteArgs& a, int h, int b, double* lds, int part) {
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
  auto knew = [&](int p) { return kn + (size_t)(p - pos) * D; };
  auto vnew = [&](int p) { return vn + (size_t)(p - pos) * D; };
  if (part == 0) {  // the summaries, when the step ends the chunk
    if (pos + lq - c0 != kChunk) return;
    T* stage = static_cast<T*>(f.k_stage) + (size_t)unit * kChunk * D;
    const int chunk = pos / kChunk;
    float* cs = f.chunk_sum + ((size_t)unit * a.r.max_chunks + chunk) * D;
    float* gs = f.group_sum + ((size_t)unit * a.r.max_chunks + chunk) * kGroups * D;
    if (pos == c0) {
      build_span<D, BF16>(c, c0, pos, pos + lq, knew, vnew, static_cast<T*>(nullptr),
                          static_cast<T*>(nullptr), cs, gs, lds);
    } else {  // earlier positions from their staging rows (written by earlier steps)
      build_span<D, BF16>(
          c, c0, c0, c0 + kChunk,
          [&](int p) { return p >= pos ? knew(p) : stage + (size_t)(p - c0) * D; },
          [&](int) { return kn; }, static_cast<T*>(nullptr), static_cast<T*>(nullptr), cs, gs, lds);
    }
    return;
  }
  // the step's tokens of group part - 1
  const int g0 = c0 + (part - 1) * kGroupTokens;
  const int lo = pos > g0 ? pos : g0;
  const int hi = pos + lq < g0 + kGroupTokens ? pos + lq : g0 + kGroupTokens;
  if (lo >= hi) return;
  T* stage = static_cast<T*>(f.k_stage) + (size_t)unit * kChunk * D;
  T* kp = c.pool8 ? nullptr : static_cast<T*>(f.k_pool) + (size_t)unit * f.pool_cap * D;
  T* vp = c.pool8 ? nullptr : static_cast<T*>(f.v_pool) + (size_t)unit * f.pool_cap * D;
  if constexpr (D == 128 && BF16) {
    if (c.pool8) {
      const Fp8Rows f8 = fp8_rows_of(f.k_pool, f.v_pool, a.r.B * c.hkv, f.pool_cap, D, unit);
      for (int p = lo; p < hi; ++p)
        fp8_append_row(c, static_cast<const uint16_t*>(f.k_new) + ((size_t)unit * lq + (p - pos)) * D,
                       static_cast<const uint16_t*>(f.v_new) + ((size_t)unit * lq + (p - pos)) * D,
                       c0, p, f8);
    }
  }
  build_span<D, BF16>(c, c0, lo, hi, knew, vnew, kp, vp, nullptr, nullptr, lds, stage);
}

template <int D, bool BF16, bool MAXQ = false, bool SPLIT = false>
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a) {
  constexpr int NV = D / 32;
  constexpr int RPP = 256 / kLanesPerRow;  // rows per pass of the workgroup
  constexpr int U = 8;                     // passes in flight
  __shared__ double s_qh[MAXQ ? kMaxHg : 1][D];  // max pooling: the heads' routing queries
  __shared__ int hist[256];
  __shared__ int kk[2];
  __shared__ double red[8];
  __shared__ int ints[8];
  extern __shared__ double dyn[];

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  if (SPLIT ? blockIdx.z >= 1 : blockIdx.z == 1) {  // a fused step's token work, per KV head
    if (h % c.kvdiv == 0) {
      if constexpr (SPLIT) step_front_part<D, BF16>(a, h / c.kvdiv, b, dyn, (int)blockIdx.z - 1);
      else step_front<D, BF16>(a, h / c.kvdiv, b, dyn);
    }
    return;
  }
  const int unit = b * c.lists + h;                     // lists and workspace: virtual sequence
  const int unit_p = (b / r.nq) * c.hkv + h / c.kvdiv;  // summaries: pool sequence, KV head

  // every load that does not depend on the position goes out first: this
  // lane's qbar slice (for level 2) and the level-1 scores (clamped to the
  // table; entries past the candidates are dropped below)
  const int sub = lane % kLanesPerRow;
  double qv[NV][4];
  if constexpr (MAXQ) {
    for (int i = tid; i < c.lhg * D; i += 256)
      s_qh[i / D][i % D] = r.qbar[(size_t)unit * c.lhg * D + i];
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qv[v][e] = r.qbar[(size_t)unit * D + 4 * (v * kLanesPerRow + sub) + e];
  }
  const double* scores = r.scores + (size_t)unit * a.score_ld;
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
      if constexpr (MAXQ) {
        d = route_row_max<NV>(gb[u], &s_qh[0][0], c.lhg, sub) * c.inv_sqrt_d;
      } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          d = fma((double)gb[u][v].x, qv[v][0], d);
          d = fma((double)gb[u][v].y, qv[v][1], d);
          d = fma((double)gb[u][v].z, qv[v][2], d);
          d = fma((double)gb[u][v].w, qv[v][3], d);
        }
        d = group8_sum_d(d) * c.inv_sqrt_d;
      }
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

// Selection for up to kFastMaxCand candidates and kFastMaxKept level-1
// chunks.  Thread t owns candidates 4t..4t+3 (so wave w owns a contiguous
// quarter of them).
//  1. Every load goes out first (scores, the per-wave score ranges that
//     route_tiles wrote, qbar, position); both levels' counts are cleared and
//     a barrier passes while the loads are in flight.  Waves 1..3 write the
//     sink, local and current groups of the list (their slots follow from the
//     position and the budgets alone).
//  2. Level 1 (sel_level, all threads): bins between the min and max of the
//     ranges, counts and member slots, a barrier, then in every wave the cut
//     and the boundary ranking.
//  3. Each wave lists its kept chunks in order (scan of the keep bits) with
//     their count; barrier.  The k1 * G group rows of the kept chunks, in
//     ascending group order, are dealt over the waves 8 rows at a time (row i
//     to wave (i / 8) % 4), every row load of a wave in flight at once; each
//     wave scores its rows into the level-2 arrays at their element index and
//     keeps the range of its scores; barrier.
//  4. Level 2 (sel_level again): thread t takes element t; the kept groups
//     are written in element order (= ascending group id) after one more
//     barrier for the per-wave counts.
constexpr int kFastMaxCand = 1024;
constexpr int kFastMaxKept = 64;  // level-1 chunks kept: level 2 ranks <= 256 groups

template <int D, bool BF16, bool MAXQ = false, bool SPLIT = false>
__global__ __launch_bounds__(256) void route_select_fast_kernel(RouteArgs a) {
  constexpr int NV = D / 32;
  constexpr int KPW = kFastMaxKept;       // kept chunks a wave can list
  // level-2 row passes per wave: 8 x 8 rows, a quarter of the kFastMaxKept * G rows
  constexpr int U = 8;
  static_assert(4 * 8 * U >= kGroups * KPW, "one pass of loads covers every level-2 row");
  __shared__ __align__(16) int s_fine[kSelBins];
  __shared__ __align__(16) int s_fine2[kSelBins];
  __shared__ __align__(16) int s_slot[kSelBins * kSelSlots];  // both levels (level 2 starts after a barrier)
  __shared__ __align__(16) double s_vals[kFastMaxCand];  // scores by element; token-plane scratch
  __shared__ int s_kl[4][KPW];             // kept candidate indices of each wave, ascending
  __shared__ double s_l2[kGroups * KPW];  // level-2 scores, ascending group order
  __shared__ int s_g2[kGroups * KPW];     // their group ids
  __shared__ int s_n2[4];                 // chunks kept by each wave
  __shared__ double s_r2[8];               // level-2 score range of each wave (min, max)
  __shared__ int s_k2[4];                  // level-2 groups kept by each wave
  __shared__ int s_nbl[2];                 // overflowed boundary members collected
  __shared__ int s_bl[kFastMaxCand];
  __shared__ double s_qh[MAXQ ? kMaxHg : 1][D];  // max pooling: the heads' routing queries

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  if (SPLIT ? blockIdx.z >= 1 : blockIdx.z == 1) {  // a fused step's token work, per KV head
    if (h % c.kvdiv == 0) {
      if constexpr (SPLIT) step_front_part<D, BF16>(a, h / c.kvdiv, b, s_vals, (int)blockIdx.z - 1);
      else step_front<D, BF16>(a, h / c.kvdiv, b, s_vals);
    }
    return;
  }
  const int unit = b * c.lists + h;                     // lists and workspace: virtual sequence
  const int unit_p = (b / r.nq) * c.hkv + h / c.kvdiv;  // summaries: pool sequence, KV head

  // ---- 1. loads (clamped into the workspace rows; unused entries ignored)
  const int sub = lane % kLanesPerRow, g8 = lane / kLanesPerRow;
  double qv[NV][4];
  if constexpr (MAXQ) {  // in LDS before the first barrier
    for (int i = tid; i < c.lhg * D; i += 256)
      s_qh[i / D][i % D] = r.qbar[(size_t)unit * c.lhg * D + i];
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qv[v][e] = r.qbar[(size_t)unit * D + 4 * (v * kLanesPerRow + sub) + e];
  }
  const double* scores = r.scores + (size_t)unit * a.score_ld;
  double x[4];
  {
    const int i0 = 4 * tid < a.score_ld - 3 ? 4 * tid : a.score_ld - 4;  // score_ld: 4 k >= 4
    const double2 p0 = *reinterpret_cast<const double2*>(scores + i0);
    const double2 p1 = *reinterpret_cast<const double2*>(scores + i0 + 2);
    x[0] = p0.x; x[1] = p0.y; x[2] = p1.x; x[3] = p1.y;
  }
  const int n_rng = a.n_tiles * 4;
  const double2 rng = reinterpret_cast<const double2*>(a.ranges)[(size_t)unit * n_rng +
                                                                 (lane < n_rng ? lane : n_rng - 1)];
  const int p0 = r.q_pos0[b];  // in flight across the barrier with the other loads
  const SelHist h1{s_fine, s_slot}, h2{s_fine2, s_slot};
  sel_clear(h1, tid, 256);
  sel_clear(h2, tid, 256);
  if (tid < 2) s_nbl[tid] = 0;
  __syncthreads();

  int pos0;
  Windows w;
  if (!route_geometry_at(c, r, a.max_cand, p0, &pos0, &w)) {
    if (tid == 0) r.n_sel[unit] = -1;
    return;
  }
  const int n_cand = w.cand_hi - w.cand_lo;
  const int ct = pos0 / kChunk;
  const int k1 = c.topk_c < n_cand ? c.topk_c : n_cand;
  const int k2 = c.topk_g < k1 * kGroups ? c.topk_g : k1 * kGroups;
  const int last = pos0 + r.lq - 1;
  const int n_head = w.sink_end * kGroups;
  const int n_tail = (ct - w.local_begin) * kGroups + (last / kGroupTokens - ct * kGroups + 1);
  int* out = r.sel + (size_t)unit * r.max_sel;
  if (wave != 0) {  // the window groups: sink | (routed) | local | current
    for (int i = tid - 64; i < n_head + n_tail; i += 192) {
      const bool head = i < n_head;
      out[head ? i : i + k2] = head ? i : w.local_begin * kGroups + (i - n_head);
    }
  }

  // ---- 2. level 1
  uint32_t keep = 0;
  if (k1 >= n_cand) {  // every candidate kept (uniform)
#pragma unroll
    for (int e = 0; e < 4; ++e) keep |= (4 * tid + e < n_cand ? 1u : 0u) << e;
  } else if (k1 > 0) {
    // range of the scores: entry l covers rows 16 l .. 16 l + 15 of the tiles
    const bool rv = lane < n_rng && 16 * lane < n_cand;
    const double mn = wave_ext_d<false>(rv ? rng.x : INFINITY);
    const double mx = wave_ext_d<true>(rv ? rng.y : -INFINITY);
    auto idx = [&](int e) { return 4 * tid + e < n_cand ? 4 * tid + e : -1; };
    // the scores by element for the boundary ranking (two 16-byte stores;
    // published by the routine's barrier)
    reinterpret_cast<double2*>(s_vals)[2 * tid] = make_double2(x[0], x[1]);
    reinterpret_cast<double2*>(s_vals)[2 * tid + 1] = make_double2(x[2], x[3]);
    keep = sel_level(x[0], x[1], x[2], x[3], idx(0), idx(1), idx(2), idx(3), 4, k1, mn, mx, s_fine,
                     s_slot, s_vals, s_bl, &s_nbl[0]);
  }

  // ---- 3. each wave's kept chunks in candidate order; one barrier; then the
  // group rows of all kept chunks in ascending group order, dealt evenly over
  // the waves (row i goes to wave (i / 8) % 4, pass i / 32)
  const int kc = __popc(keep);
  const int kincl = wave_incl_scan(kc);
  {
    int o = kincl - kc;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((keep >> e) & 1u) s_kl[wave][o++] = 4 * tid + e;
  }
  if (lane == 63) s_n2[wave] = kincl;  // chunks kept by this wave
  __syncthreads();
  const int c0 = s_n2[0], c01 = c0 + s_n2[1], c012 = c01 + s_n2[2];
  const int n2 = (c012 + s_n2[3]) * kGroups;  // = k1 * G <= 256
  double mn2 = INFINITY, mx2 = -INFINITY;
  if (n2 > 0) {  // uniform
    float4 gb[U][NV];
    int gids[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int i = 32 * u + 8 * wave + g8;
      i = i < n2 ? i : n2 - 1;  // clamped: every load issues, extras ignored
      const int j = i / kGroups;  // kept chunk rank, ascending candidate order
      const int rg = (j >= c0) + (j >= c01) + (j >= c012);
      const int e = j - (rg == 0 ? 0 : rg == 1 ? c0 : rg == 2 ? c01 : c012);
      gids[u] = (w.cand_lo + s_kl[rg][e]) * kGroups + i % kGroups;
      const float4* rowp = reinterpret_cast<const float4*>(
          r.group_sum + ((size_t)unit_p * r.max_chunks * kGroups + gids[u]) * D);
#pragma unroll
      for (int v = 0; v < NV; ++v) gb[u][v] = rowp[v * kLanesPerRow + sub];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (32 * u + 8 * wave >= n2) break;  // uniform: no row of this pass is in the list
      const int i = 32 * u + 8 * wave + g8;
      double d = 0.0;
      if constexpr (MAXQ) {
        d = route_row_max<NV>(gb[u], &s_qh[0][0], c.lhg, sub) * c.inv_sqrt_d;
      } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          d = fma((double)gb[u][v].x, qv[v][0], d);
          d = fma((double)gb[u][v].y, qv[v][1], d);
          d = fma((double)gb[u][v].z, qv[v][2], d);
          d = fma((double)gb[u][v].w, qv[v][3], d);
        }
        d = group8_sum_d(d) * c.inv_sqrt_d;
      }
      if (sub == 0 && i < n2) {
        s_l2[i] = d;
        s_g2[i] = gids[u];
        mn2 = fmin(mn2, d);
        mx2 = fmax(mx2, d);
      }
    }
  }
  mn2 = wave_ext_d<false>(mn2);
  mx2 = wave_ext_d<true>(mx2);
  if (lane == 0) {
    s_r2[wave] = mn2;
    s_r2[4 + wave] = mx2;
  }
  __syncthreads();

  // ---- 4. level 2: thread t takes element t (ascending group order)
  double y = 0.0;
  int gid = 0;
  if (tid < n2) {
    y = s_l2[tid];
    gid = s_g2[tid];
  }
  bool kept2 = tid < n2;
  if (k2 < n2 && k2 > 0) {  // uniform
    const double mn = fmin(fmin(s_r2[0], s_r2[1]), fmin(s_r2[2], s_r2[3]));
    const double mx = fmax(fmax(s_r2[4], s_r2[5]), fmax(s_r2[6], s_r2[7]));
    kept2 = sel_level(y, 0.0, 0.0, 0.0, tid < n2 ? tid : -1, -1, -1, -1, 1, k2, mn, mx, s_fine2,
                      s_slot, s_l2, s_bl, &s_nbl[1]) & 1u;
  } else if (k2 <= 0) {
    kept2 = false;
  }
  // the kept groups in element order = ascending group id
  const unsigned long long m = __ballot(kept2);
  if (lane == 0) s_k2[wave] = __popcll(m);
  __syncthreads();
  if (kept2) {
    int off = lanes_below(m);
    for (int v = 0; v < wave; ++v) off += s_k2[v];
    out[n_head + off] = gid;
  }
  if (tid == 0) r.n_sel[unit] = n_head + k2 + n_tail;
}

// The fast selection applies when every unit has at most kFastMaxCand
// candidates and level 1 keeps at most kFastMaxKept chunks.
static bool fast_select(const KCfg& cfg, int max_cand) {
  return max_cand <= kFastMaxCand && cfg.topk_c <= kFastMaxKept;
}

static int max_cand_of(const KCfg& cfg, int max_chunks) {
  return max_chunks > cfg.n_sink ? max_chunks - cfg.n_sink : 1;
}

// Workspace per unit: level-1 scores (row stride rounded up to 4), the pooled
// query, and the score range of every 16 rows (wave) of every tile.
static int score_ld_of(int max_cand) { return (max_cand + 3) / 4 * 4; }
static int n_tiles_of(int max_cand) { return (max_cand + kTile - 1) / kTile; }

int route_score_ld(const KCfg& cfg, int max_chunks) {
  return score_ld_of(max_cand_of(cfg, max_chunks));
}

// Pooled-query rows per unit: one, or one per query head with max pooling.
static int qbar_rows(const KCfg& cfg) { return cfg.route_max ? cfg.lhg : 1; }

size_t route_ws_bytes(const KCfg& cfg, int B, int max_chunks) {
  const int mc = max_cand_of(cfg, max_chunks);
  return (size_t)B * cfg.lists *
         (score_ld_of(mc) + (size_t)qbar_rows(cfg) * cfg.d + 8 * n_tiles_of(mc)) * sizeof(double);
}

size_t route_select_lds(const KCfg& cfg, int max_chunks) {
  const int max_cand = max_cand_of(cfg, max_chunks);
  if (fast_select(cfg, max_cand)) return 0;  // static LDS only
  const int n2 = cfg.topk_c * kGroups;
  const size_t nmax = (size_t)(max_cand > n2 ? max_cand : n2);
  return nmax * (sizeof(double) + 3 * sizeof(int)) + (size_t)n2 * sizeof(int);
}

template <int D, bool BF16, bool MAXQ>
static void launch_tiles(bool multi, bool pooled_once, dim3 grid, hipStream_t st,
                         const RouteArgs& a) {
  if (pooled_once) {  // pooled query once per unit, then the tiles
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 2, MAXQ>), dim3(1, grid.y, grid.z), dim3(256), 0, st, a);
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 3, MAXQ>), grid, dim3(256), 0, st, a);
  } else if (multi) {
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 1, MAXQ>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((route_tiles_kernel<D, BF16, 0, MAXQ>), grid, dim3(256), 0, st, a);
  }
}

// Tiles then selection for one (head dim, dtype, pooling); split: the token
// work of a step of many tokens on kFrontParts workgroups per unit (such
// steps run at head_dim 128 in bf16 only).
template <int D, bool BF16, bool MAXQ>
static void launch_route_d(bool multi, bool pooled_once, bool fast, bool split, dim3 grid,
                           dim3 sgrid, size_t lds, hipStream_t st, const RouteArgs& a) {
  launch_tiles<D, BF16, MAXQ>(multi, pooled_once, grid, st, a);
  if constexpr (D == 128 && BF16) {
    if (split) {
      if (fast) hipLaunchKernelGGL((route_select_fast_kernel<D, BF16, MAXQ, true>), sgrid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((route_select_kernel<D, BF16, MAXQ, true>), sgrid, dim3(256), lds, st, a);
      return;
    }
  }
  if (fast) hipLaunchKernelGGL((route_select_fast_kernel<D, BF16, MAXQ>), sgrid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((route_select_kernel<D, BF16, MAXQ>), sgrid, dim3(256), lds, st, a);
}

hipError_t launch_route(const KCfg& cfg, const RouteLaunch& r, hipStream_t st,
                        const StepFront* front) {
  RouteArgs a{};
  a.cfg = cfg;
  a.r = r;
  a.max_cand = max_cand_of(cfg, r.max_chunks);
  a.score_ld = score_ld_of(a.max_cand);
  a.n_tiles = n_tiles_of(a.max_cand);
  // the workspace holds the scores with stride score_ld, then qbar, then the
  // ranges (the callers place qbar at B * lists * score_ld)
  a.ranges = r.qbar + (size_t)r.B * cfg.lists * qbar_rows(cfg) * cfg.d;
  if (front) a.f = *front;
  const int n_tiles = a.n_tiles;
  size_t lds = route_select_lds(cfg, r.max_chunks);
  const size_t front_lds = (size_t)256 * 2 * sizeof(double);  // build_span scratch: S*P*2 doubles
  if (front && lds < front_lds) lds = front_lds;
  dim3 grid(n_tiles, cfg.lists, r.B);
  // the token work: one workgroup per unit, or kFrontParts for a step of
  // many tokens
  const bool split = front && r.lq >= kFrontSplitLq && cfg.d == 128 && cfg.dtype == HGA_BF16;
  dim3 sgrid(cfg.lists, r.B, front ? (split ? 1 + kFrontParts : 2) : 1);
  const bool bf = cfg.dtype == HGA_BF16;
  const bool multi = r.lq > 256 / (cfg.d / 2);  // more tokens than slices
  const bool fast = fast_select(cfg, a.max_cand);
  const bool mq = cfg.route_max != 0;
  if (cfg.d == 128) {
    if (bf) {
      if (mq) launch_route_d<128, true, true>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
      else launch_route_d<128, true, false>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
    } else {
      if (mq) launch_route_d<128, false, true>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
      else launch_route_d<128, false, false>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
    }
  } else {
    if (bf) {
      if (mq) launch_route_d<64, true, true>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
      else launch_route_d<64, true, false>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
    } else {
      if (mq) launch_route_d<64, false, true>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
      else launch_route_d<64, false, false>(multi, r.pool_once, fast, split, grid, sgrid, lds, st, a);
    }
  }
  return hipGetLastError();
}

}  // namespace hga
