// Block scores on CDNA4 (gfx950).
//
// What is computed ([UP] "drop" and "block-wise estimation" paragraphs; [CP] causal
// mask over absolute positions): for every window row (query head h, window row j
// at absolute position t) the softmax over keys 0..t of scale * q.k, summed over
// heads, rows and the G keys of each block, normalised per request.
//
// How: one pass over the keys on the matrix cores instead of the two-pass
// max-then-sum that an online softmax usually takes.  For each (row, block) the
// kernel keeps the block-local maximum m_b and the block-local sum
// l_b = sum_{k in b} 2^(x_k - m_b) (x = logit * scale * log2 e).  Row statistics
// (m, l) follow by the usual online-softmax merge, and a block's mass is
// sum_rows 2^(m_b - m) * l_b / l -- the same quantity, rearranged.  This reads K
// once and runs Q K^T once, half the matrix-core work and key traffic of two passes.
//
// Kernels (all launched on the caller's stream, in this order):
//   up_score_plan_kernel     per-request offsets from the device cu_seqlens, checked
//                            against the host-derived totals
//   up_score_partial_kernel  Q K^T on bf16 MFMA (32x32x16), per-(row, block) (m_b, l_b)
//                            and per-(row, key chunk) merged statistics
//   up_row_stats_kernel      merge chunk statistics into per-row (m, l)
//   up_block_mass_kernel     per-block mass, float64 sums in a fixed order
//   up_normalize_kernel      per-request normalisation to scores that sum to one
#include "up_internal.h"

#include <math.h>

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax merge of (m, s) into (M, S), both in log2 units: afterwards
// S * 2^M = S_old * 2^M_old + s * 2^m.  An empty side has m = -inf, s = 0.
__device__ __forceinline__ void merge_ml(float& M, float& S, float m, float s) {
  if (m > M) {
    S = S * fast_exp2(M - m) + s;   // M = -inf gives 0 * 0 + s
    M = m;
  } else if (m != kNegInf) {
    S += s * fast_exp2(m - M);
  }
}

// Number of requests whose work items end at or before x, i.e. the request holding
// work item x.  Every lane of the wave must call it (wave-wide ballot).
__device__ __forceinline__ int request_of_item(const ReqPlan* __restrict__ plan, int B, int x) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int base = 0; base < B; base += 64) {
    const int i = base + lane;
    const bool pred = (i < B) && (plan[i].item_end <= x);
    cnt += __popcll(__ballot(pred));
  }
  return cnt;
}

// ---------------------------------------------------------------------------
// Plan
// ---------------------------------------------------------------------------
__global__ void up_score_plan_kernel(const int32_t* __restrict__ cu, ScoreShape s, Totals host,
                                     WsHeader* __restrict__ hdr, ReqPlan* __restrict__ plan,
                                     int* __restrict__ err) {
  if (threadIdx.x != 0) return;
  const int gs = s.Hq / s.Hkv;
  bool ok = (cu[0] == 0);
  int64_t win = 0, blk = 0, items = 0, mlp = 0, csp = 0;
  for (int i = 0; i < s.B; ++i) {
    const int32_t a = cu[i], b = cu[i + 1];
    int64_t L = (int64_t)b - a;
    if (L < 0) { ok = false; L = 0; }
    const int64_t W = L < s.n ? L : s.n;
    const int64_t nb = (L + s.G - 1) / s.G;
    const int64_t nch = (nb + s.CB - 1) / s.CB;
    const int64_t R = gs * W;
    const int64_t nrt = (R + s.rows_wg - 1) / s.rows_wg;
    items += nch * s.Hkv * nrt;
    ReqPlan p;
    p.tok_off = a; p.L = (int32_t)L; p.W = (int32_t)W; p.win_off = (int32_t)win;
    p.blk_off = (int32_t)blk; p.nb = (int32_t)nb; p.nch = (int32_t)nch;
    p.item_end = (int32_t)items; p.ml_off = mlp; p.cs_off = csp;
    plan[i] = p;
    win += W; blk += nb; mlp += nb * s.Hkv * R; csp += nch * s.Hkv * R;
  }
  ok = ok && (int64_t)cu[s.B] == host.T && win == host.win_rows && blk == host.nb_tot &&
       items == host.items && mlp == host.ml_pairs && csp == host.cs_pairs;
  hdr->valid = ok ? 1 : 0;
  if (!ok) atomicOr(err, 1);
}

// ---------------------------------------------------------------------------
// Partial statistics on the matrix cores
//
// Workgroup = 8 waves = one (request, kv head g, query-row tile, key chunk).
// Each wave holds QT tiles of 32 query rows of kv head g's group in VGPRs as the B
// operand (rows r = j * gs + hh: window row j, head g*gs + hh).  Key tiles of
// UK = 32*KT keys are staged through LDS (double-buffered, padded rows) and read as
// the A operand, so S^T = K Q^T lands with one query per lane column: lane l and
// lane l^32 together hold all keys of a tile for query l%32, and the per-query
// max and sum over a block are in-lane reductions plus one cross-half exchange.
//
// The head dimension is contracted in a permuted order that both operands share:
// lane half h, k-step s holds d-elements [h*D/2 + 8s, h*D/2 + 8s + 8), so every
// lane reads one contiguous D-byte run per row.
// ---------------------------------------------------------------------------
template <int D, int QT, int KT>
__global__ __launch_bounds__(512, 1) void up_score_partial_kernel(
    const uint16_t* __restrict__ qwin, const uint16_t* __restrict__ kmat,
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq, int Hkv,
    int G, int CB, float c, float2* __restrict__ ml, float2* __restrict__ cs) {
  constexpr int NT = 512;
  constexpr int UK = KT * 32;          // keys per LDS stage
  constexpr int RS = 2 * D + 16;       // LDS bytes per key row (16 B pad against bank conflicts)
  constexpr int SEGS = UK * D / 8;     // 16-byte segments per stage
  constexpr int SPT = (SEGS + NT - 1) / NT;
  constexpr int DS = D / 16;           // MFMA k-steps over the head dimension
  constexpr int ROWS = 8 * QT * 32;    // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * UK * RS];

  if (hdr->valid != 1) return;
  const int x = blockIdx.x;
  const int i = request_of_item(plan, B, x);
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  const int gs = Hq / Hkv;
  const int R = gs * pr.W;
  const int nrt = (R + ROWS - 1) / ROWS;
  int xl = x - (i > 0 ? plan[i - 1].item_end : 0);
  const int g = xl % Hkv;
  xl /= Hkv;
  const int rt = xl % nrt;
  const int ch = xl / nrt;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int row0 = rt * ROWS + wave * (QT * 32);

  // Query operand, resident for the whole chunk.
  bf16x8 qreg[QT][DS];
  int qpos[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int r = row0 + t * 32 + l32;
    if (r < R) {
      const int j = r / gs, hh = r - j * gs;
      const uint16_t* src =
          qwin + ((int64_t)(pr.win_off + j) * Hq + g * gs + hh) * D + half * (D / 2);
#pragma unroll
      for (int s = 0; s < DS; ++s) qreg[t][s] = *reinterpret_cast<const bf16x8*>(src + s * 8);
      qpos[t] = pr.L - pr.W + j;
    } else {
#pragma unroll
      for (int s = 0; s < DS; ++s) qreg[t][s] = bf16x8{};
      qpos[t] = -1;   // inactive row: every key masked in masked stages, never stored
    }
  }

  const int b0 = ch * CB;
  const int b1 = min(pr.nb, b0 + CB);
  const int k0 = b0 * G;
  const int kend = min(b1 * G, pr.L);
  const int nunits = (kend - k0 + UK - 1) / UK;
  const int upb = G / UK;
  const int64_t kstride = (int64_t)Hkv * D;
  const uint16_t* kbase = kmat + ((int64_t)pr.tok_off * Hkv + g) * D;
  const int fast_limit = pr.L - pr.W;   // keys <= this are visible to every window row

  uint4 pre[SPT];
  auto gload = [&](int u) {
    const int ks = k0 + u * UK;
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
      const int e = tid + q * NT;
      if (SEGS % NT == 0 || e < SEGS) {
        const int key = e / (D / 8), part = e % (D / 8);
        const int kabs = ks + key;
        pre[q] = (kabs < pr.L)
                     ? *reinterpret_cast<const uint4*>(kbase + (int64_t)kabs * kstride + part * 8)
                     : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
      const int e = tid + q * NT;
      if (SEGS % NT == 0 || e < SEGS) {
        const int key = e / (D / 8), part = e % (D / 8);
        *reinterpret_cast<uint4*>(lds + buf * UK * RS + key * RS + part * 16) = pre[q];
      }
    }
  };

  float mb[QT], lb[QT], Mc[QT], Lc[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) { mb[t] = kNegInf; lb[t] = 0.f; Mc[t] = kNegInf; Lc[t] = 0.f; }

  const int t_st = (QT == 2) ? half : 0;          // the tile this lane stores
  const int r_st = row0 + t_st * 32 + l32;
  const bool st_ok = (QT == 2 || half == 0) && (r_st < R);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int u = 0; u < nunits; ++u) {
    if (u + 1 < nunits) gload(u + 1);
    const uint8_t* kb = lds + (u & 1) * UK * RS;
    f32x16 acc[KT][QT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int t = 0; t < QT; ++t) acc[kt][t] = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(kb + (kt * 32 + l32) * RS + half * D + s * 16);
#pragma unroll
        for (int t = 0; t < QT; ++t)
          acc[kt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[t][s], acc[kt][t], 0, 0, 0);
      }
    }

    const int ks = k0 + u * UK;
    const bool masked = (ks + UK - 1 > fast_limit);   // uniform across the workgroup
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (masked) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            // 32x32 MFMA result layout: register e of lane l holds row
            // 8*(e/4) + 4*(l/32) + e%4 (the key) and column l%32 (the query).
            const int key = ks + kt * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            if (key > qpos[t]) acc[kt][t][e] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[kt][t][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m = mx * c;                          // exact max of the scaled logits
      const float msub = (mx == kNegInf) ? 0.f : m;    // all masked: every term is 2^-inf = 0
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += fast_exp2(fmaf(acc[kt][t][e], c, -msub));
      sum += __shfl_xor(sum, 32);                      // same value on both halves
      merge_ml(mb[t], lb[t], m, sum);
    }

    const int uu = (ks - k0) / UK;                     // stage index within the chunk
    const bool block_end = (uu % upb == upb - 1) || (u == nunits - 1);
    if (block_end) {
      const int bl = b0 + uu / upb;                    // request-local block
      if (st_ok) {
        const float mv = (QT == 2 && t_st) ? mb[QT - 1] : mb[0];
        const float lv = (QT == 2 && t_st) ? lb[QT - 1] : lb[0];
        ml[pr.ml_off + ((int64_t)bl * Hkv + g) * R + r_st] = make_float2(mv, lv);
      }
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        merge_ml(Mc[t], Lc[t], mb[t], lb[t]);
        mb[t] = kNegInf;
        lb[t] = 0.f;
      }
    }
    if (u + 1 < nunits) lstore((u + 1) & 1);
    __syncthreads();
  }

  if (st_ok) {
    const float mv = (QT == 2 && t_st) ? Mc[QT - 1] : Mc[0];
    const float lv = (QT == 2 && t_st) ? Lc[QT - 1] : Lc[0];
    cs[pr.cs_off + ((int64_t)ch * Hkv + g) * R + r_st] = make_float2(mv, lv);
  }
}

// ---------------------------------------------------------------------------
// Row statistics: merge the key chunks of every (request, kv head, row).
// Output layout: rs[win_off*Hq + g*R + r] (the request's Hq*W rows, g-major).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int request_of_row(const ReqPlan* __restrict__ plan, int B, int Hq,
                                              int64_t x) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)(plan[mid].win_off + plan[mid].W) * Hq <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void up_row_stats_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq, int Hkv,
    const float2* __restrict__ cs, float2* __restrict__ rs, int64_t total_rows) {
  if (hdr->valid != 1) return;
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= total_rows) return;
  const int i = request_of_row(plan, B, Hq, x);
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  const int R = (Hq / Hkv) * pr.W;
  const int64_t local = x - (int64_t)pr.win_off * Hq;   // = g*R + r
  const int g = (int)(local / R), r = (int)(local % R);
  float M = kNegInf, S = 0.f;
  for (int chk = 0; chk < pr.nch; ++chk) {
    const float2 v = cs[pr.cs_off + ((int64_t)chk * Hkv + g) * R + r];
    merge_ml(M, S, v.x, v.y);
  }
  rs[x] = make_float2(M, S);
}

// ---------------------------------------------------------------------------
// Block masses: mass[b] = sum_{g, r} 2^(m_b - m) * l_b / l, float64, fixed order.
// One workgroup per global block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int request_of_block(const ReqPlan* __restrict__ plan, int B,
                                                int64_t x) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)plan[mid].blk_off + plan[mid].nb <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int w = NT / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void up_block_mass_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq,
    const float2* __restrict__ ml, const float2* __restrict__ rs, double* __restrict__ mass) {
  __shared__ double red[256];
  if (hdr->valid != 1) return;
  const int64_t blk = blockIdx.x;
  const int i = request_of_block(plan, B, blk);
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  const int64_t b = blk - pr.blk_off;
  const int64_t terms = (int64_t)Hq * pr.W;           // Hkv * R
  const float2* mrow = ml + pr.ml_off + b * terms;
  const float2* rrow = rs + (int64_t)pr.win_off * Hq;
  double acc = 0.0;
  for (int64_t e = threadIdx.x; e < terms; e += 256) {
    const float2 v = mrow[e];
    const float2 w = rrow[e];
    acc += (double)v.y * (double)fast_exp2(v.x - w.x) / (double)w.y;
  }
  const double tot = block_sum_f64<256>(acc, red);
  if (threadIdx.x == 0) mass[blk] = tot;
}

// ---------------------------------------------------------------------------
// Normalise: scores[b] = mass[b] / sum of the request's masses.  One workgroup
// per request; the sum has a fixed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void up_normalize_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B,
    const double* __restrict__ mass, float* __restrict__ scores) {
  __shared__ double red[256];
  if (hdr->valid != 1) return;
  const int i = blockIdx.x;
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  double acc = 0.0;
  for (int b = threadIdx.x; b < pr.nb; b += 256) acc += mass[pr.blk_off + b];
  const double tot = block_sum_f64<256>(acc, red);
  for (int b = threadIdx.x; b < pr.nb; b += 256)
    scores[pr.blk_off + b] = (float)(mass[pr.blk_off + b] / tot);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
ScoreWs score_ws_layout(int B, const Totals& t) {
  ScoreWs L;
  size_t off = align_up(sizeof(WsHeader));
  L.plan = off; off = align_up(off + (size_t)B * sizeof(ReqPlan));
  L.ml = off;   off = align_up(off + (size_t)t.ml_pairs * sizeof(float2));
  L.cs = off;   off = align_up(off + (size_t)t.cs_pairs * sizeof(float2));
  L.rs = off;   off = align_up(off + (size_t)t.rows * sizeof(float2));
  L.mass = off; off = align_up(off + (size_t)t.nb_tot * sizeof(double));
  L.total = off;
  return L;
}

static inline char* wsb(void* ws) { return static_cast<char*>(ws); }

hipError_t launch_score_plan(const int32_t* cu, const ScoreShape& s, const Totals& t, void* ws,
                             const ScoreWs& L, int* err, hipStream_t st) {
  hipLaunchKernelGGL(up_score_plan_kernel, dim3(1), dim3(64), 0, st, cu, s, t,
                     reinterpret_cast<WsHeader*>(wsb(ws)),
                     reinterpret_cast<ReqPlan*>(wsb(ws) + L.plan), err);
  return hipGetLastError();
}

template <int D, int QT, int KT>
static hipError_t launch_partial_t(const void* qwin, const void* k, const ScoreShape& s,
                                   const Totals& t, void* ws, const ScoreWs& L, float c,
                                   hipStream_t st) {
  hipLaunchKernelGGL((up_score_partial_kernel<D, QT, KT>), dim3((unsigned)t.items), dim3(512), 0,
                     st, static_cast<const uint16_t*>(qwin), static_cast<const uint16_t*>(k),
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B, s.Hq, s.Hkv, s.G,
                     s.CB, c, reinterpret_cast<float2*>(wsb(ws) + L.ml),
                     reinterpret_cast<float2*>(wsb(ws) + L.cs));
  return hipGetLastError();
}

hipError_t launch_score_partial(const void* qwin, const void* k, const ScoreShape& s,
                                const Totals& t, void* ws, const ScoreWs& L, float c,
                                hipStream_t st) {
  if (t.items == 0) return hipSuccess;
  const int key = s.d * 100 + s.qt * 10 + s.kt;
  switch (key) {
    case 6421: return launch_partial_t<64, 2, 1>(qwin, k, s, t, ws, L, c, st);
    case 6422: return launch_partial_t<64, 2, 2>(qwin, k, s, t, ws, L, c, st);
    case 12821: return launch_partial_t<128, 2, 1>(qwin, k, s, t, ws, L, c, st);
    case 12822: return launch_partial_t<128, 2, 2>(qwin, k, s, t, ws, L, c, st);
    case 25611: return launch_partial_t<256, 1, 1>(qwin, k, s, t, ws, L, c, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_row_stats(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                            hipStream_t st) {
  if (t.rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((t.rows + 255) / 256);
  hipLaunchKernelGGL(up_row_stats_kernel, dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B, s.Hq, s.Hkv,
                     reinterpret_cast<const float2*>(wsb(ws) + L.cs),
                     reinterpret_cast<float2*>(wsb(ws) + L.rs), t.rows);
  return hipGetLastError();
}

hipError_t launch_block_mass(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                             hipStream_t st) {
  if (t.nb_tot == 0) return hipSuccess;
  hipLaunchKernelGGL(up_block_mass_kernel, dim3((unsigned)t.nb_tot), dim3(256), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B, s.Hq,
                     reinterpret_cast<const float2*>(wsb(ws) + L.ml),
                     reinterpret_cast<const float2*>(wsb(ws) + L.rs),
                     reinterpret_cast<double*>(wsb(ws) + L.mass));
  return hipGetLastError();
}

hipError_t launch_normalize(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                            float* scores, hipStream_t st) {
  if (s.B == 0 || t.nb_tot == 0) return hipSuccess;
  hipLaunchKernelGGL(up_normalize_kernel, dim3(s.B), dim3(256), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B,
                     reinterpret_cast<const double*>(wsb(ws) + L.mass), scores);
  return hipGetLastError();
}

}  // namespace up
