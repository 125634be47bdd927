// The layer that runs on the surviving tokens ([UP] "propagation" and "Sparsity
// Propagation" paragraphs: after a drop every later sub-layer, attention and FFN,
// computes on the kept tokens only; "scheduler" paragraph: the survivors keep their
// original positions).
//
//   up_attn_plan_kernel    per-request padded offsets and workgroup tiles, checked
//                          against the host's totals;
//   up_rope_layout_kernel  rotary embedding of q and k at the carried positions
//                          (float64 rotation, rounded once to bfloat16) into
//                          head-major, 64-row padded copies, and v transposed to
//                          [kv head][d][token] for the P V product;
//   up_attention_kernel    causal GQA flash attention on the matrix cores;
//   up_swiglu_kernel       silu(gate) * up for the FFN.
// The FFN and projection GEMMs are plain bf16 GEMMs; they are served by hipBLASLt in
// the separate layer library (gemm.hip).
#include "attn_geom.h"
#include "up_dpp.h"
#include "up_internal.h"


#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

namespace up {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Plan: padded offsets po[i] (64-row aligned start of request i in the rotated
// copies) and workgroup-tile offsets tp[i] (tiles of tok_tile tokens), both as
// exclusive prefix sums; valid = 1 only when the device cu_seqlens gives the same
// totals the host sized the launch with.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;

// With n > 0 also the window slots: k_i = the tiles of request i that hold some of its
// last W = min(n, L) rows (its first slots, heaviest first), wp = their prefix.
__global__ __launch_bounds__(kPlanThreads) void up_attn_plan_kernel(
    const int32_t* __restrict__ cu, int B, int tok_tile, int n, int64_t R_h, int64_t Rp_h,
    int64_t tiles_h, int64_t wtiles_h, WsHeader* __restrict__ hdr, int32_t* __restrict__ po,
    int32_t* __restrict__ tp, int32_t* __restrict__ wp, int* __restrict__ err) {
  constexpr int NWV = kPlanThreads / 64;
  __shared__ uint64_t wsum[3][NWV];
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) bad = 0;
  __syncthreads();
  uint64_t carry_p = 0, carry_t = 0, carry_w = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int i = base + tid;
    uint32_t lp = 0, nt = 0, nw = 0;
    if (i < B) {
      const int32_t a = cu[i], b = cu[i + 1];
      if (b < a || (i == 0 && a != 0)) bad = 1;
      const uint32_t L = b >= a ? (uint32_t)(b - a) : 0u;
      lp = (L + 63u) & ~63u;
      nt = (L + (uint32_t)tok_tile - 1u) / (uint32_t)tok_tile;
      if (n > 0 && L > 0) {
        const uint32_t W = L < (uint32_t)n ? L : (uint32_t)n;
        nw = nt - (L - W) / (uint32_t)tok_tile;
      }
    }
    const uint64_t sp = wave_scan_u64(lp), sn = wave_scan_u64(nt);   // inclusive
    const uint64_t sw = wave_scan_u64(nw);
    if (lane == 63) {
      wsum[0][wave] = sp;
      wsum[1][wave] = sn;
      wsum[2][wave] = sw;
    }
    __syncthreads();
    uint64_t op = 0, on = 0, ow = 0, tot_p = 0, tot_n = 0, tot_w = 0;
    for (int w = 0; w < NWV; ++w) {
      if (w < wave) {
        op += wsum[0][w];
        on += wsum[1][w];
        ow += wsum[2][w];
      }
      tot_p += wsum[0][w];
      tot_n += wsum[1][w];
      tot_w += wsum[2][w];
    }
    if (i < B) {
      po[i] = (int32_t)(carry_p + op + sp - lp);
      tp[i] = (int32_t)(carry_t + on + sn - nt);
      wp[i] = (int32_t)(carry_w + ow + sw - nw);
    }
    carry_p += tot_p;
    carry_t += tot_n;
    carry_w += tot_w;
    __syncthreads();
  }
  if (tid == 0) {
    po[B] = (int32_t)carry_p;
    tp[B] = (int32_t)carry_t;
    wp[B] = (int32_t)carry_w;
    const bool ok = !bad && (B == 0 || (int64_t)cu[B] == R_h) && (int64_t)carry_p == Rp_h &&
                    (int64_t)carry_t == tiles_h && (int64_t)carry_w == wtiles_h;
    hdr->valid = ok ? 1 : 0;
    if (!ok) atomicOr(err, 1);
  }
}

using attn::request_of;

// ---------------------------------------------------------------------------
// Rotary embedding and layout.  One workgroup per 64 padded rows.  Pair (i, i + d/2)
// of a head turns by pos * theta^(-2i/d); the angle, its sine and cosine and the
// rotation are float64, and the result is rounded to bfloat16 once (round to odd
// into float32, then to nearest even into bfloat16, which is the correct rounding
// of the float64 value).  Padding rows are zero.
//   qr [Hq][Rp][d], kr [Hkv][Rp][d]    rotated copies
//   vt [Hkv][d][Rp]                    v transposed; within each 16-token group
//                                      token bits 2 and 3 are swapped, so the keys a
//                                      lane contracts in one MFMA step are adjacent
//   kn [Hkv][Rp / 64]                  (when kn is given) the largest norm of the 64
//                                      rotated bf16 key rows of each kv head and tile
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t bf16_of_f64(double x) {
  const float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) u |= 1u;   // sticky bit: round to odd
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ double f64_of_bf16(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

using attn::swap_bits23;

template <int D>
__global__ __launch_bounds__(256) void up_rope_layout_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos,
    const WsHeader* __restrict__ hdr, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ po, int B, int Hq, int Hkv, int64_t Rp, double log2_theta,
    uint16_t* __restrict__ qr, uint16_t* __restrict__ kr, uint16_t* __restrict__ vt,
    float* __restrict__ kn) {
  constexpr int PG = D / 8;          // groups of 4 pairs per row
  constexpr int NU = 64 * PG / 256;  // (row, group) items per thread
  constexpr int VRS = 2 * D + 4;     // LDS bytes per v row (padded against bank conflicts)
  __shared__ __attribute__((aligned(16))) uint8_t vs[64 * VRS];
  __shared__ uint32_t knorm2[kMaxAttnKvHeads];   // per kv head: largest |k'|^2 (float bits)
  if (hdr->valid != 1) return;
  const int64_t row0p = (int64_t)blockIdx.x * 64;
  const int i = request_of(po, B, row0p);
  const int t0 = (int)(row0p - po[i]);
  const int L = cu[i + 1] - cu[i];
  const int tid = threadIdx.x;
  const bool norms = kn != nullptr;   // the host passes kn only when Hkv <= kMaxAttnKvHeads
  if (norms) {
    for (int h = tid; h < Hkv; h += 256) knorm2[h] = 0u;
    __syncthreads();
  }

  // q and k: each thread owns NU (row, 4-pair group) items and their 8 angles, taken
  // NC at a time so that the float64 angles of a chunk fit beside everything else.
  constexpr int NC = NU < 4 ? NU : 4;
  const int Hs = Hq + Hkv;
#pragma unroll 1
  for (int u0 = 0; u0 < NU; u0 += NC) {
    double cs[NC][4], sn[NC][4];
    int64_t src_row[NC];   // packed token row, -1 for padding
    int rr_of[NC], pg_of[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int item = tid + 256 * (u0 + u);
      const int rr = item / PG, pg = item % PG;
      rr_of[u] = rr;
      pg_of[u] = pg;
      const int t = t0 + rr;
      src_row[u] = t < L ? (int64_t)cu[i] + t : -1;
      const double p = src_row[u] >= 0 ? (double)pos[src_row[u]] : 0.0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ip = 4 * pg + m;
        const double inv_freq = exp2(-(2.0 * ip / D) * log2_theta);
        sincos(p * inv_freq, &sn[u][m], &cs[u][m]);
      }
    }
    for (int hs = 0; hs < Hs; ++hs) {
      const bool isq = hs < Hq;
      const int hh = isq ? hs : hs - Hq;
      const int H = isq ? Hq : Hkv;
      const uint16_t* src = isq ? q : k;
      uint16_t* dst = (isq ? qr : kr) + ((int64_t)hh * Rp + row0p) * D;
      float rowmax = 0.f;   // keys: largest squared norm of this thread's rows
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        ushort4 lo = make_ushort4(0, 0, 0, 0), hi = make_ushort4(0, 0, 0, 0);
        if (src_row[u] >= 0) {
          const uint16_t* sp = src + (src_row[u] * H + hh) * D + 4 * pg_of[u];
          const ushort4 xl = *reinterpret_cast<const ushort4*>(sp);
          const ushort4 xh = *reinterpret_cast<const ushort4*>(sp + D / 2);
          const uint16_t al[4] = {xl.x, xl.y, xl.z, xl.w};
          const uint16_t ah[4] = {xh.x, xh.y, xh.z, xh.w};
          uint16_t rl[4], rh[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const double a = f64_of_bf16(al[m]), b = f64_of_bf16(ah[m]);
            rl[m] = bf16_of_f64(a * cs[u][m] - b * sn[u][m]);
            rh[m] = bf16_of_f64(b * cs[u][m] + a * sn[u][m]);
          }
          lo = make_ushort4(rl[0], rl[1], rl[2], rl[3]);
          hi = make_ushort4(rh[0], rh[1], rh[2], rh[3]);
        }
        uint16_t* dd = dst + (int64_t)rr_of[u] * D + 4 * pg_of[u];
        *reinterpret_cast<ushort4*>(dd) = lo;
        *reinterpret_cast<ushort4*>(dd + D / 2) = hi;
        if (norms && !isq) {
          // squared norm of the rotated bf16 key row: its PG items sit in adjacent lanes
          const uint16_t v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          float ss = 0.f;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const float f = __uint_as_float((uint32_t)v8[m] << 16);
            ss = fmaf(f, f, ss);
          }
#pragma unroll
          for (int off = PG / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
          rowmax = fmaxf(rowmax, ss);
        }
      }
      // non-negative floats order as their bit patterns
      if (norms && !isq) atomicMax(&knorm2[hh], __float_as_uint(rowmax));
    }
  }
  if (norms) {
    __syncthreads();
    for (int h = tid; h < Hkv; h += 256)
      kn[(int64_t)h * (Rp / 64) + blockIdx.x] = sqrtf(__uint_as_float(knorm2[h]));
  }

  // v: stage 64 rows of one kv head in LDS, then write 16-byte runs of 8 tokens per
  // d-row in the swapped token order.
  constexpr int RCH = D / 8;                 // 16-byte chunks per v row
  constexpr int WCH = D * 8;                 // 16-byte output chunks per head (D rows x 8)
  for (int g = 0; g < Hkv; ++g) {
    __syncthreads();
    for (int c = tid; c < 64 * RCH; c += 256) {
      const int rr = c / RCH, ch = c % RCH;
      const int t = t0 + rr;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (t < L) val = *reinterpret_cast<const uint4*>(v + (((int64_t)cu[i] + t) * Hkv + g) * D + 8 * ch);
      uint32_t* dw = reinterpret_cast<uint32_t*>(vs + rr * VRS + 16 * ch);
      dw[0] = val.x;
      dw[1] = val.y;
      dw[2] = val.z;
      dw[3] = val.w;
    }
    __syncthreads();
    for (int c = tid; c < WCH; c += 256) {
      const int dv = c / 8, ch = c % 8;
      uint16_t e[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int tok = swap_bits23(8 * ch + m);   // token stored at position 8 ch + m
        e[m] = *reinterpret_cast<const uint16_t*>(vs + tok * VRS + 2 * dv);
      }
      uint4 o;
      o.x = e[0] | ((uint32_t)e[1] << 16);
      o.y = e[2] | ((uint32_t)e[3] << 16);
      o.z = e[4] | ((uint32_t)e[5] << 16);
      o.w = e[6] | ((uint32_t)e[7] << 16);
      *reinterpret_cast<uint4*>(vt + ((int64_t)g * D + dv) * Rp + row0p + 8 * ch) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Causal GQA flash attention on the matrix cores.
//
// Workgroup = 4 waves (one per SIMD) = HQ query heads x TT 32-token tiles of one kv
// head (HQ * TT = 4), one wave per (head, tile), its 32 query rows held as the B
// operand in VGPRs.  Keys and values stream through a ring of four LDS stages of 32
// tokens (K tile [32][d] and V^T tile [d][32], 16-byte granules XOR-swizzled), copied
// global -> LDS directly.
//   S^T = K Q^T        (keys as rows: each lane column is one query, so a query's
//                       softmax statistics are in-lane plus one lane-pair exchange)
//   O^T += V^T P^T     (P^T straight from the S^T registers, rounded to bf16; the
//                       keys a lane holds are the ones its V^T operand reads,
//                       because v was stored in that order)
// Softmax: one reference Rs per query in log2 units; P = 2^(x - Rs) with x the
// scaled logit.  Rs moves only when a stage's maximum exceeds it by more than 32 (a
// wave-uniform branch that rescales O and l), so P <= 2^32 and no per-stage rescale
// of O is needed.  A stage's body issues the next stage's S^T before its own softmax,
// so those MFMAs overlap the VALU work; a wave's diagonal stage (its last) is masked
// before its maximum is taken.  Up to d = 128 a workgroup takes 64 KiB of LDS and at
// most 256 registers per lane, so two workgroups share a CU (two waves per SIMD); at
// d = 256 the stage is 32 KiB and the O accumulator alone 128 registers, one
// workgroup per CU.  Workgroups are ordered heaviest tile first; with the kv head in
// blockIdx.x the workgroups of one kv head share an XCD's L2 when Hkv * quads is a
// multiple of 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
}

// vmcnt(N) and lgkmcnt(0), then a workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  asm volatile("s_barrier" ::: "memory");
}

constexpr float kRebase = 32.f;

// Window-row block statistics (the fused form of the block scores).  A wave whose
// rows reach the last W = min(n, L) tokens of its request sums, per lane, the
// probabilities 2^(x - Rs) of each G-key block beside its softmax (bsum, rescaled with
// l and O when Rs moves); at a block's end (or at the wave's last 32-key half-step) the
// two lanes of a window row add their halves and one of them stores (Rs, block sum)
// for that (row, block).  Blocks wholly after the wave's diagonal tile hold no key the
// row may see: they get (-inf, 0).  At the end the row's (Rs, 1 / l) and, when asked,
// its natural-log log-sum-exp are stored.  Pairs and rows use the score pass's layouts:
// pair (b, e) at ml_off + b Hq W + e and row e at win_off Hq + e, with
// e = g gs W + w gs + (head - g gs) for window row w of query head head (gs = Hq / Hkv).
struct WinStats {
  bool wave = false;   // some row of the wave is a window row (wave-uniform)
  bool row = false;    // this lane's row is a window row
  float bsum = 0.f;
  float2* pair0 = nullptr;   // this row's pair of block 0
  float2* rsp = nullptr;
  float* lsep = nullptr;
  int64_t terms = 0;
  int nb = 0, G = 64;
  int pend = 0;   // statistics stores since the newest stage copies (wave-uniform)

  // The wave's rows are the tokens [first_row_tok, first_row_tok + 32); it keeps
  // statistics when one of them is a window row, so every flush has lanes that store.
  __device__ __forceinline__ void init(const AttnScoreOut& so, int i, int L, int g, int head,
                                       int Hq, int Hkv, bool wact, int first_row_tok, int qtok) {
    if (!wact || so.hdr->valid != 1) return;
    const ReqPlan pr = so.plan[i];
    const int wfirst = L - pr.W;
    wave = first_row_tok + 31 >= wfirst && first_row_tok < L;
    if (!wave) return;
    const int gs = Hq / Hkv;
    row = qtok >= wfirst && qtok < L;
    const int wr = row ? qtok - wfirst : 0;
    terms = (int64_t)Hq * pr.W;
    const int64_t e = attn::win_term(g, gs, pr.W, wr, head);
    pair0 = so.ml + pr.ml_off + e;
    rsp = so.rs + (int64_t)pr.win_off * Hq + e;
    lsep = so.row_lse ? so.row_lse + ((int64_t)pr.win_off + wr) * Hq + head : nullptr;
    nb = pr.nb;
    G = so.G;
  }
  // After the P V of half-step hs (keys [32 hs, 32 hs + 32)); last = the wave's last.
  // A half-step wholly past the request's last key (the padded end of its last 64-token
  // tile) can lie in block nb: nothing is stored for it (its probabilities are zero).
  __device__ __forceinline__ void flush(int hs, int last, float Rs, int half) {
    if (!wave || !attn::stats_flush(hs, last, G)) return;
    const float tot = pair_sum(bsum);
    const int b = attn::stats_block(hs, G);
    if (b < nb) {
      // a window wave always has lanes with row && half == 0, so the store is issued
      if (row && half == 0) pair0[(int64_t)b * terms] = make_float2(Rs, tot);
      ++pend;
      asm volatile("" ::: "memory");   // the store stays ahead of the next wait
    }
    bsum = 0.f;
  }
  __device__ __forceinline__ void finish(int last, float Rs, float l, int half) {
    if (!wave || !row || half != 0) return;
    for (int b = attn::stats_tail_first(last, G); b < nb; ++b)
      pair0[(int64_t)b * terms] = make_float2(kNegInf, 0.f);
    *rsp = make_float2(Rs, 1.f / l);
    if (lsep) *lsep = (Rs + log2f(l)) * 0.6931471805599453f;
  }
};

template <int D, bool ST>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void up_attention_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vt, const WsHeader* __restrict__ hdr,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ po,
    const int32_t* __restrict__ tp, int B, int Hq, int Hkv, int HQ, int TT, int64_t Rp,
    float c, uint16_t* __restrict__ out, AttnScoreOut so, int mode,
    const int32_t* __restrict__ wp) {
  using G = attn::W4<D>;
  constexpr int NS = G::NS, DS = G::DS, DT = G::DT, VRB = G::VRB, SB = G::SB, KSPT = G::KSPT,
                VSPT = G::VSPT, SPT = G::SPT;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * SB];

  if (hdr->valid != 1) {
    if constexpr (ST)
      if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) so.hdr->valid = 0;
    return;
  }
  // 32-token tiles (tile_shift 5): a workgroup's stages are 32 keys each.
  const attn::Wg w = attn::wg_of(blockIdx.x, blockIdx.y, Hq, Hkv, HQ, TT, B, cu, po, tp, mode,
                                 wp, 5);
  const int i = w.i, L = w.L, g = w.g, nst = w.nst;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5,
            l32 = lane & 31;
  const attn::Wv wv = attn::wave4_of(w, wave, Hq, Hkv, HQ);
  const int head = wv.head;
  const int tw = wv.tw;   // this wave's 32-token tile (its diagonal stage)
  const bool wact = wv.act;

  // Query operand (one 32-row tile), the head dimension in the permuted order both
  // operands share: lane half h, k-step s covers d-elements [h D/2 + 8 s, +8).
  bf16x8 qreg[DS];
  if (wact) {
    const uint16_t* src = qr + attn::q_src4<D>(w, wv, l32, half, Rp);
#pragma unroll
    for (int s = 0; s < DS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(src + s * 8);
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qreg[s] = bf16x8{};
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): only stage copies from here

  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8*)lds;
  auto issue = [&](int st) {
    const uint32_t sb = lds_base + (uint32_t)((st & (NS - 1)) * SB);
    const uint16_t* kst = kr + attn::k_stage4<D>(w, st, Rp);
#pragma unroll
    for (int q = 0; q < KSPT; ++q)
      lds_dma16(kst + G::k_src(q, tid), __builtin_amdgcn_readfirstlane(sb + G::k_dst(q, wave)));
    const uint16_t* vst = vt + attn::v_stage4<D>(w, st, Rp);
#pragma unroll
    for (int q = 0; q < VSPT; ++q)
      lds_dma16(vst + G::v_src(q, tid, Rp),
                __builtin_amdgcn_readfirstlane(sb + G::v_dst(q, wave)));
  };

  uint32_t krd[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) krd[s] = G::k_rd(l32, half, s);
  // V^T row dt * 32 + l32 has the swizzle of l32 (dt * 32 is a multiple of 16 rows).
  uint32_t vrd[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) vrd[jj] = G::v_rd(l32, 2 * jj + half);

  float Rs = 0.f, lsum = 0.f;
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x16{};
  const int qtok = attn::query_token4(wv, l32);
  WinStats ws;
  if constexpr (ST) ws.init(so, i, L, g, head, Hq, Hkv, wact, tw * 32, qtok);

  // S^T of stage (= half-step) hs into acc.
  auto s_mfma = [&](int hs, f32x16& acc) {
    const uint8_t* sl = lds + (hs & (NS - 1)) * SB;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sl + krd[s]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], s == 0 ? f32x16{} : acc, 0, 0, 0);
    }
  };
  // Causal mask of the diagonal stage (keys past the query -> -inf).
  auto mask = [&](int hs, f32x16& acc) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (attn::acc_key(hs, e, half) > qtok) acc[e] = kNegInf;
    }
  };
  auto rebase = [&](const f32x16& acc, bool init) {
    float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      m0 = fmaxf(m0, acc[e]);
      m1 = fmaxf(m1, acc[e + 1]);
    }
    const float mx = pair_max(fmaxf(m0, m1)) * c;
    const bool need = init || mx > Rs + kRebase;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      if (init) {
        Rs = mx;
      } else {
        const float rn = fmaxf(Rs, mx);
        const float sc = __builtin_amdgcn_exp2f(Rs - rn);
        lsum *= sc;
        if constexpr (ST) ws.bsum *= sc;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] *= sc;
        Rs = rn;
      }
    }
  };
  // Softmax of stage hs (S^T in acc) and O^T += V^T P^T over its 32 keys.
  auto pv = [&](int hs, const f32x16& acc) {
    const uint8_t* sl = lds + (hs & (NS - 1)) * SB;
    bf16x8 va[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        va[dt][jj] = *reinterpret_cast<const bf16x8*>(sl + dt * 32 * VRB + vrd[jj]);
    f32x16 p;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      p[e] = __builtin_amdgcn_exp2f(fmaf(acc[e], c, -Rs));
      p[e + 1] = __builtin_amdgcn_exp2f(fmaf(acc[e + 1], c, -Rs));
      s0 += p[e];
      s1 += p[e + 1];
    }
    lsum += s0 + s1;
    if constexpr (ST) ws.bsum += s0 + s1;
    const bf16x8 pb[2] = {__builtin_convertvector(p.lo, bf16x8),
                          __builtin_convertvector(p.hi, bf16x8)};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][jj], pb[jj], O[dt], 0, 0, 0);
  };

  // Ring: while body(st) reads stages st and st+1, stages st+2 and st+3 are in flight.
  // Before body(st): wait for stage st+1 (stage st+2, issued earlier, may stay in
  // flight), publish it with a barrier -- after which every wave is done with stage
  // st-1 -- and refill that slot with stage st+3.
  auto sync_for = [&](int st) {
    if (st + 1 >= nst) return;
    if (st + 2 < nst) {
      // Stores share the vector-memory count with the stage copies and complete in issue
      // order with them: the block-statistics stores issued since the newest copies are
      // younger than them, so the wait leaves those stores and the newest stage in flight.
      if constexpr (ST) {
        if (ws.pend == 2) wait_barrier<SPT + 2>();
        else if (ws.pend == 1) wait_barrier<SPT + 1>();
        else wait_barrier<SPT>();
      } else {
        wait_barrier<SPT>();
      }
    } else {
      wait_barrier<0>();
    }
    if (st + 3 < nst) {
      issue(st + 3);
      if constexpr (ST) ws.pend = 0;
    }
  };

  issue(0);
  if (nst > 1) issue(1);
  if (nst > 2) issue(2);
  if (nst > 2) wait_barrier<2 * SPT>();
  else if (nst > 1) wait_barrier<SPT>();
  else wait_barrier<0>();

  f32x16 accA, accB;
  if (wact) {
    s_mfma(0, accA);
    if (tw == 0) mask(0, accA);
    rebase(accA, true);
  }
  // cur holds S^T of stage hs; nxt receives stage hs+1's (waited for by the caller).
  auto body = [&](int hs, f32x16& cur, f32x16& nxt) {
    if (!wact || hs > tw) return;
    if (hs + 1 < tw) {
      s_mfma(hs + 1, nxt);
      pv(hs, cur);
      if constexpr (ST) ws.flush(hs, tw, Rs, half);
      rebase(nxt, false);
    } else if (hs + 1 == tw) {
      s_mfma(hs + 1, nxt);
      pv(hs, cur);
      if constexpr (ST) ws.flush(hs, tw, Rs, half);
      mask(hs + 1, nxt);
      rebase(nxt, false);
    } else {
      pv(hs, cur);
      if constexpr (ST) ws.flush(hs, tw, Rs, half);
    }
  };
  for (int st = 0; st < nst; st += 2) {
    sync_for(st);
    body(st, accA, accB);
    if (st + 1 < nst) {
      sync_for(st + 1);
      body(st + 1, accB, accA);
    }
  }

  if (!wact) return;
  const float lt = pair_sum(lsum), inv = 1.f / lt;
  if constexpr (ST) ws.finish(tw, Rs, lt, half);
  if (qtok >= L) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int eg = 0; eg < 4; ++eg) {
      const int dv = dt * 32 + 8 * eg + 4 * half;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4 o4 = {O[dt][4 * eg] * inv, O[dt][4 * eg + 1] * inv, O[dt][4 * eg + 2] * inv,
                        O[dt][4 * eg + 3] * inv};
      *reinterpret_cast<bf16x4*>(out + attn::out_index4<D>(cu, w, wv, l32, Hq, dv)) =
          __builtin_convertvector(o4, bf16x4);
    }
}

// ---------------------------------------------------------------------------
// The same attention with 8 waves per workgroup sharing one ring of 64-key stages
// (d = 64 and 128, at most kMaxAttnKvHeads kv heads).  Workgroup = HQ query heads x
// TT 64-token tiles of one kv head (HQ * TT = 4), two waves per (head, tile), 32
// query rows per wave; two waves per SIMD, one workgroup per CU (128 KiB of LDS at
// d = 128).  Every K and V^T stage is copied once for 256 query rows instead of 128,
// and a stage costs one barrier per 64 keys instead of per 32.  A 64-key stage is two
// half-steps of 32 keys (row tiles kt = 0, 1 of the K tile and granules 4 kt .. 4 kt
// + 3 of the V^T rows).  Before a half-step's rebase check the wave compares a bound
// on its logits -- the largest query norm of the wave times the stage's largest key
// norm (kn, from the layout pass) times c -- with its references: when no logit can
// exceed a reference by the rebase margin the check cannot fire and is skipped, so the
// results are those of the unconditional check.  All addresses come from attn_geom.h.
// ---------------------------------------------------------------------------
template <int D, bool ST>
__global__ __launch_bounds__(512, 1) void up_attention_w8_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vt, const WsHeader* __restrict__ hdr,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ po,
    const int32_t* __restrict__ tp, const float* __restrict__ kn, int B, int Hq, int Hkv,
    int HQ, int TT, int64_t Rp, float c, uint16_t* __restrict__ out, AttnScoreOut so, int mode,
    const int32_t* __restrict__ wp) {
  using G = attn::W8<D>;
  constexpr int NS = G::NS, DS = G::DS, DT = G::DT, SB = G::SB, SPT = G::SPT;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * SB];

  if (hdr->valid != 1) {
    // no attention: the block statistics are not written either, so the block masses
    // after this kernel must not run on them
    if constexpr (ST)
      if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) so.hdr->valid = 0;
    return;
  }
  const attn::Wg w = attn::wg_of(blockIdx.x, blockIdx.y, Hq, Hkv, HQ, TT, B, cu, po, tp, mode,
                                 wp);
  const int nst = w.nst;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5,
            l32 = lane & 31;
  const attn::Wv wv = attn::wave_of(w, wave, Hq, Hkv, HQ);
  const int tw = wv.tw;
  const bool wact = wv.act;

  // Query operand: lane half h, k-step s covers d-elements [h D/2 + 8 s, +8).
  bf16x8 qreg[DS];
  if (wact) {
    const uint16_t* src = qr + attn::q_src<D>(w, wv, l32, half, Rp);
#pragma unroll
    for (int s = 0; s < DS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(src + s * 8);
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qreg[s] = bf16x8{};
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): only stage copies from here

  // Largest query norm of the wave times c (float32 norms and the MFMA's float32 sums
  // are far inside the 0.1% margin).
  float qbound;
  {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)qreg[s][e];
        ss = fmaf(f, f, ss);
      }
    float m = pair_sum(ss);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    qbound = __builtin_amdgcn_readfirstlane(sqrtf(m) * c * 1.001f);
  }

  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8*)lds;
  auto issue = [&](int st) {
    const uint32_t sb = lds_base + (uint32_t)((st & (NS - 1)) * SB);
    const uint16_t* kst = kr + attn::k_stage<D>(w, st, Rp);
#pragma unroll
    for (int q = 0; q < G::KSPT; ++q)
      lds_dma16(kst + G::k_src(q, tid), __builtin_amdgcn_readfirstlane(sb + G::k_dst(q, wave)));
    const uint16_t* vst = vt + attn::v_stage<D>(w, st, Rp);
#pragma unroll
    for (int q = 0; q < G::VSPT; ++q)
      lds_dma16(vst + G::v_src(q, tid, Rp),
                __builtin_amdgcn_readfirstlane(sb + G::v_dst(q, wave)));
  };

  uint32_t krd[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) krd[s] = G::k_rd(l32, half, s);
  uint32_t vrd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vrd[j] = G::v_rd(l32, 2 * j + half);

  float Rs = 0.f, lsum = 0.f;
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x16{};
  const int qtok = attn::query_token(wv, l32);
  WinStats ws;
  if constexpr (ST) ws.init(so, w.i, w.L, w.g, wv.head, Hq, Hkv, wact, attn::query_token(wv, 0),
                            qtok);

  // S^T of half-step hs (keys [32 hs, 32 hs + 32): stage hs / 2, row tile hs % 2).
  auto s_mfma = [&](int hs, f32x16& acc) {
    const uint8_t* sl = lds + ((hs >> 1) & (NS - 1)) * SB + (hs & 1) * 32 * G::KRB;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sl + krd[s]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], s == 0 ? f32x16{} : acc, 0, 0, 0);
    }
  };
  auto mask = [&](int hs, f32x16& acc) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (attn::acc_key(hs, e, half) > qtok) acc[e] = kNegInf;
  };
  auto rebase = [&](const f32x16& acc, bool init) {
    float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      m0 = fmaxf(m0, acc[e]);
      m1 = fmaxf(m1, acc[e + 1]);
    }
    const float mx = pair_max(fmaxf(m0, m1)) * c;
    const bool need = init || mx > Rs + kRebase;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      if (init) {
        Rs = mx;
      } else {
        const float rn = fmaxf(Rs, mx);
        const float sc = __builtin_amdgcn_exp2f(Rs - rn);
        lsum *= sc;
        if constexpr (ST) ws.bsum *= sc;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] *= sc;
        Rs = rn;
      }
    }
  };
  // True when no logit of half-step hs can exceed the wave's references by kRebase.
  auto bound_ok = [&](int hs) {
    const float b = qbound * kn[attn::kn_index(w, hs >> 1, Rp)] - kRebase;
    return __builtin_amdgcn_ballot_w64(b > Rs) == 0;
  };
  auto pv = [&](int hs, const f32x16& acc) {
    const int kt = hs & 1;
    const uint8_t* sl = lds + ((hs >> 1) & (NS - 1)) * SB;
    bf16x8 va[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        va[dt][jj] = *reinterpret_cast<const bf16x8*>(sl + dt * 32 * G::VRB + vrd[2 * kt + jj]);
    f32x16 p;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      p[e] = __builtin_amdgcn_exp2f(fmaf(acc[e], c, -Rs));
      p[e + 1] = __builtin_amdgcn_exp2f(fmaf(acc[e + 1], c, -Rs));
      s0 += p[e];
      s1 += p[e + 1];
    }
    lsum += s0 + s1;
    if constexpr (ST) ws.bsum += s0 + s1;
    const bf16x8 pb[2] = {__builtin_convertvector(p.lo, bf16x8),
                          __builtin_convertvector(p.hi, bf16x8)};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][jj], pb[jj], O[dt], 0, 0, 0);
  };

  // Ring: stages st+1 and st+2 in flight while st is consumed; stage st+1 is waited
  // for (and published by a barrier, after which every wave is done with stage st-1)
  // before the second half of stage st, whose body issues the S^T of stage st+1's
  // first half; then stage st-1's slot is refilled with stage st+3.
  auto sync_for = [&](int st) {
    if (st + 1 >= nst) return;
    if (st + 2 < nst) {
      // Stores share the vector-memory count with the stage copies and complete in issue
      // order with them: the block-statistics stores issued since the newest copies are
      // younger than them, so the wait leaves those stores and the newest stage in flight.
      if constexpr (ST) {
        if (ws.pend == 2) wait_barrier<SPT + 2>();
        else if (ws.pend == 1) wait_barrier<SPT + 1>();
        else wait_barrier<SPT>();
      } else {
        wait_barrier<SPT>();
      }
    } else {
      wait_barrier<0>();
    }
    if (st + 3 < nst) {
      issue(st + 3);
      if constexpr (ST) ws.pend = 0;
    }
  };

  issue(0);
  if (nst > 1) issue(1);
  if (nst > 2) issue(2);
  if (nst > 2) wait_barrier<2 * SPT>();
  else if (nst > 1) wait_barrier<SPT>();
  else wait_barrier<0>();

  const int last_hs = 2 * tw + 1;   // the wave's last half-step (end of its diagonal stage)
  f32x16 accA, accB;
  if (wact) {
    s_mfma(0, accA);
    if (tw == 0) mask(0, accA);
    rebase(accA, true);
  }
  // cur holds S^T of half-step hs; nxt receives half-step hs+1's.
  auto body = [&](int hs, f32x16& cur, f32x16& nxt) {
    if (!wact || hs > last_hs) return;
    if (hs + 1 < 2 * tw) {            // next half-step is before the diagonal stage
      const bool skip = bound_ok(hs + 1);
      s_mfma(hs + 1, nxt);
      pv(hs, cur);
      if constexpr (ST) ws.flush(hs, last_hs, Rs, half);
      if (!skip) rebase(nxt, false);
    } else if (hs + 1 <= last_hs) {   // next half-step is in the diagonal stage
      const bool skip = bound_ok(hs + 1);
      s_mfma(hs + 1, nxt);
      pv(hs, cur);
      if constexpr (ST) ws.flush(hs, last_hs, Rs, half);
      mask(hs + 1, nxt);
      if (!skip) rebase(nxt, false);
    } else {
      pv(hs, cur);
      if constexpr (ST) ws.flush(hs, last_hs, Rs, half);
    }
  };
  for (int st = 0; st < nst; ++st) {
    body(2 * st, accA, accB);
    sync_for(st);
    body(2 * st + 1, accB, accA);
  }

  if (!wact) return;
  const float lt = pair_sum(lsum), inv = 1.f / lt;
  if constexpr (ST) ws.finish(last_hs, Rs, lt, half);
  if (qtok >= w.L) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int eg = 0; eg < 4; ++eg) {
      const int dv = dt * 32 + 8 * eg + 4 * half;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4 o4 = {O[dt][4 * eg] * inv, O[dt][4 * eg + 1] * inv, O[dt][4 * eg + 2] * inv,
                        O[dt][4 * eg + 3] * inv};
      *reinterpret_cast<bf16x4*>(out + attn::out_index<D>(cu, w, wv, l32, Hq, dv)) =
          __builtin_convertvector(o4, bf16x4);
    }
}

// ---------------------------------------------------------------------------
// SwiGLU gate: a[r][j] = silu(gu[r][j]) * gu[r][F + j] in float32, rounded to
// bfloat16.  Eight columns per thread, grid-stride.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void up_swiglu_kernel(const uint16_t* __restrict__ gu,
                                                        int64_t R, int F,
                                                        uint16_t* __restrict__ a) {
  const int64_t per_row = F / 8;
  const int64_t n = R * per_row;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = x / per_row, c8 = (x - r * per_row) * 8;
    const bf16x8 gv = *reinterpret_cast<const bf16x8*>(gu + r * 2 * F + c8);
    const bf16x8 uv = *reinterpret_cast<const bf16x8*>(gu + r * 2 * F + F + c8);
    const f32x8 gf = __builtin_convertvector(gv, f32x8);
    const f32x8 uf = __builtin_convertvector(uv, f32x8);
    f32x8 o;
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = gf[m] / (1.f + __expf(-gf[m])) * uf[m];
    *reinterpret_cast<bf16x8*>(a + r * F + c8) = __builtin_convertvector(o, bf16x8);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
AttnWs attn_ws_layout(int B, int Hq, int Hkv, int d, int64_t Rp) {
  AttnWs w;
  size_t o = 0;
  w.hdr = o;
  o += align_up(sizeof(WsHeader));
  w.po = o;
  o += align_up(sizeof(int32_t) * (size_t)(B + 1));
  w.tp = o;
  o += align_up(sizeof(int32_t) * (size_t)(B + 1));
  w.wp = o;
  o += align_up(sizeof(int32_t) * (size_t)(B + 1));
  w.qr = o;
  o += align_up((size_t)Hq * Rp * d * 2);
  w.kr = o;
  o += align_up((size_t)Hkv * Rp * d * 2);
  w.vt = o;
  o += align_up((size_t)Hkv * Rp * d * 2);
  w.kn = o;
  if (attn_w8(d, Hkv)) o += align_up((size_t)Hkv * (Rp / 64) * sizeof(float));
  w.total = o;
  return w;
}

hipError_t launch_attn_plan(const int32_t* cu, const AttnShape& s, void* ws, const AttnWs& L,
                            int* err, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  hipLaunchKernelGGL(up_attn_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, cu, s.B,
                     attn_tile_tokens(s.d, s.Hkv) * s.TT, s.n, s.R, s.Rp, s.tiles, s.wtiles,
                     reinterpret_cast<WsHeader*>(w + L.hdr),
                     reinterpret_cast<int32_t*>(w + L.po), reinterpret_cast<int32_t*>(w + L.tp),
                     reinterpret_cast<int32_t*>(w + L.wp), err);
  return hipGetLastError();
}

hipError_t launch_rope_layout(const void* q, const void* k, const void* v, const int32_t* pos,
                              const int32_t* cu, const AttnShape& s, void* ws, const AttnWs& L,
                              double log2_theta, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const auto* hdr = reinterpret_cast<const WsHeader*>(w + L.hdr);
  const auto* po = reinterpret_cast<const int32_t*>(w + L.po);
  auto* qr = reinterpret_cast<uint16_t*>(w + L.qr);
  auto* kr = reinterpret_cast<uint16_t*>(w + L.kr);
  auto* vt = reinterpret_cast<uint16_t*>(w + L.vt);
  auto* kn = attn_w8(s.d, s.Hkv) ? reinterpret_cast<float*>(w + L.kn) : nullptr;
  const dim3 grid((unsigned)(s.Rp / 64));
  auto kq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto kv = static_cast<const uint16_t*>(v);
  if (s.d == 64)
    hipLaunchKernelGGL(up_rope_layout_kernel<64>, grid, dim3(256), 0, st, kq, kk, kv, pos, hdr, cu,
                       po, s.B, s.Hq, s.Hkv, s.Rp, log2_theta, qr, kr, vt, kn);
  else if (s.d == 128)
    hipLaunchKernelGGL(up_rope_layout_kernel<128>, grid, dim3(256), 0, st, kq, kk, kv, pos, hdr,
                       cu, po, s.B, s.Hq, s.Hkv, s.Rp, log2_theta, qr, kr, vt, kn);
  else
    hipLaunchKernelGGL(up_rope_layout_kernel<256>, grid, dim3(256), 0, st, kq, kk, kv, pos, hdr,
                       cu, po, s.B, s.Hq, s.Hkv, s.Rp, log2_theta, qr, kr, vt, kn);
  return hipGetLastError();
}

template <bool ST>
static void launch_attention_kernels(const AttnShape& s, dim3 grid, hipStream_t st,
                                     const uint16_t* qr, const uint16_t* kr, const uint16_t* vt,
                                     const WsHeader* hdr, const int32_t* cu, const int32_t* po,
                                     const int32_t* tp, const int32_t* wp, const float* kn,
                                     float c, uint16_t* o, const AttnScoreOut& so, int mode) {
  if (attn_w8(s.d, s.Hkv)) {
    if (s.d == 64)
      hipLaunchKernelGGL((up_attention_w8_kernel<64, ST>), grid, dim3(512), 0, st, qr, kr, vt,
                         hdr, cu, po, tp, kn, s.B, s.Hq, s.Hkv, s.HQ, s.TT, s.Rp, c, o, so, mode,
                         wp);
    else
      hipLaunchKernelGGL((up_attention_w8_kernel<128, ST>), grid, dim3(512), 0, st, qr, kr, vt,
                         hdr, cu, po, tp, kn, s.B, s.Hq, s.Hkv, s.HQ, s.TT, s.Rp, c, o, so, mode,
                         wp);
    return;
  }
  if (s.d == 64)
    hipLaunchKernelGGL((up_attention_kernel<64, ST>), grid, dim3(256), 0, st, qr, kr, vt, hdr,
                       cu, po, tp, s.B, s.Hq, s.Hkv, s.HQ, s.TT, s.Rp, c, o, so, mode, wp);
  else if (s.d == 128)
    hipLaunchKernelGGL((up_attention_kernel<128, ST>), grid, dim3(256), 0, st, qr, kr, vt, hdr,
                       cu, po, tp, s.B, s.Hq, s.Hkv, s.HQ, s.TT, s.Rp, c, o, so, mode, wp);
  else
    hipLaunchKernelGGL((up_attention_kernel<256, ST>), grid, dim3(256), 0, st, qr, kr, vt, hdr,
                       cu, po, tp, s.B, s.Hq, s.Hkv, s.HQ, s.TT, s.Rp, c, o, so, mode, wp);
}

hipError_t launch_attention(const int32_t* cu, const AttnShape& s, void* ws, const AttnWs& L,
                            float c, void* out, hipStream_t st, const AttnScoreOut* so,
                            int mode) {
  char* w = static_cast<char*>(ws);
  const auto* hdr = reinterpret_cast<const WsHeader*>(w + L.hdr);
  const auto* po = reinterpret_cast<const int32_t*>(w + L.po);
  const auto* tp = reinterpret_cast<const int32_t*>(w + L.tp);
  const auto* wp = reinterpret_cast<const int32_t*>(w + L.wp);
  const auto* qr = reinterpret_cast<const uint16_t*>(w + L.qr);
  const auto* kr = reinterpret_cast<const uint16_t*>(w + L.kr);
  const auto* vt = reinterpret_cast<const uint16_t*>(w + L.vt);
  const auto* kn = attn_w8(s.d, s.Hkv) ? reinterpret_cast<const float*>(w + L.kn) : nullptr;
  const int64_t slots = mode == attn::kSlotsAll      ? s.tiles
                        : mode == attn::kSlotsWindow ? s.wtiles
                                                     : s.tiles - s.wtiles;
  if (slots == 0) return hipSuccess;
  const dim3 grid((unsigned)(s.Hkv * (s.Hq / s.Hkv / s.HQ)), (unsigned)slots);
  auto o = static_cast<uint16_t*>(out);
  if (so)
    launch_attention_kernels<true>(s, grid, st, qr, kr, vt, hdr, cu, po, tp, wp, kn, c, o, *so,
                                   mode);
  else
    launch_attention_kernels<false>(s, grid, st, qr, kr, vt, hdr, cu, po, tp, wp, kn, c, o,
                                    AttnScoreOut{}, mode);
  return hipGetLastError();
}

hipError_t launch_swiglu(const void* gu, int64_t R, int F, void* a, hipStream_t st) {
  const int64_t n = R * (F / 8);
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 64);
  hipLaunchKernelGGL(up_swiglu_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(gu), R, F, static_cast<uint16_t*>(a));
  return hipGetLastError();
}

}  // namespace up
