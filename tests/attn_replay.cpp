// Host replay of the attention kernels' addressing (block_wise_token_amd/csrc/
// consumer.hip: up_attention_w8_kernel for d = 64 and 128 up to 256 kv heads,
// up_attention_kernel, the 4-wave kernel, otherwise), built with g++ against the same
// index functions the kernels call (attn_geom.h).  No GPU code runs here.
//
//   attn_replay D Hq Hkv L0,L1,... [n G]
//
// Parts 1 and 2 run for the kernel that serves the shape (W8 or W4).
// Part 1 (per head dimension, every lane): the global-to-LDS copies of a stage fill
// the stage's K and V^T tiles exactly once, inside the stage; every K operand read
// returns the key and head-dimension elements the query operand of the same lane and
// k-step holds; every V^T operand read returns the head-dimension row and the keys the
// lane's P^T register holds (through the stored token order); the accumulator layout
// and the output stores cover each head-dimension element once.
// Part 2 (the launch): for every workgroup and wave, the request, tiles and stages;
// the ring's hand-over (a stage is read only after the wait and barrier that complete
// it, and its slot is refilled only after the barrier that follows its last read);
// the mask leaving exactly the causal keys; and every global access (K and V^T copies,
// query loads, key-norm entries, output stores) inside its buffer and inside the
// request's padded rows; every output element of every real row written once.
// Part 3 (with n and G): the window-row block statistics the kernels store when asked
// (up_rope_attention_scores): for every window row and query head, with the wave's
// half-steps as either kernel runs them (64-token tiles of two 32-key half-steps in the
// 8-wave kernel, 32-token tiles in the 4-wave kernel), every block of the request gets
// exactly one (reference, sum) pair, inside the request's pairs, and the row's
// statistics and log-sum-exp land inside their arrays.
// Prints "ok" and exits 0, or prints the first violation and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <string>
#include <vector>

#include "attn_geom.h"

namespace {

[[noreturn]] void fail(const char* what, long long a = 0, long long b = 0, long long c = 0) {
  std::printf("FAIL: %s (%lld, %lld, %lld)\n", what, a, b, c);
  std::exit(1);
}
#define CHECK(cond, ...) \
  do {                   \
    if (!(cond)) fail(#cond, ##__VA_ARGS__); \
  } while (0)

// What one 16-byte LDS granule of a stage holds after the copies.
struct Gran {
  int kind = -1;   // 0 = K, 1 = V^T
  int a = -1;      // K: key in the stage; V^T: head-dimension row
  int b = -1;      // K: element offset in the row (multiple of 8); V^T: stored position of
                   //    the first of 8 tokens
};

template <int D>
void part1() {
  using G = up::attn::W8<D>;
  const int ngran = G::SB / 16;
  std::vector<Gran> map(ngran);
  std::vector<int> kcov(64 * D / 8, 0), vcov(D * 64 / 8, 0);
  for (int q = 0; q < G::KSPT; ++q)
    for (int tid = 0; tid < G::NT; ++tid) {
      const int wave = tid / 64, lane = tid % 64;
      const uint32_t dst = G::k_dst(q, wave) + 16u * lane;
      CHECK(dst % 16 == 0 && dst + 16 <= (uint32_t)G::KB, q, tid, dst);
      const int src = G::k_src(q, tid);
      CHECK(src % 8 == 0 && src >= 0 && src + 8 <= 64 * D, q, tid, src);
      CHECK(map[dst / 16].kind == -1, q, tid, dst);
      map[dst / 16] = Gran{0, src / D, src % D};
      kcov[src / 8]++;
    }
  for (int q = 0; q < G::VSPT; ++q)
    for (int tid = 0; tid < G::NT; ++tid) {
      const int wave = tid / 64, lane = tid % 64;
      const uint32_t dst = G::v_dst(q, wave) + 16u * lane;
      CHECK(dst % 16 == 0 && dst >= (uint32_t)G::KB && dst + 16 <= (uint32_t)G::SB, q, tid, dst);
      // the V^T source offset is row * Rp + token; replay with a row pitch of 64 tokens
      // (that of one stage) and also check the token part stays inside the stage
      const int64_t Rp = 1 << 20;
      const int64_t src = G::v_src(q, tid, Rp);
      const int row = (int)(src / Rp), tok = (int)(src % Rp);
      CHECK(row >= 0 && row < D && tok % 8 == 0 && tok + 8 <= 64, q, tid, src);
      CHECK(map[dst / 16].kind == -1, q, tid, dst);
      map[dst / 16] = Gran{1, row, tok};
      vcov[(row * 64 + tok) / 8]++;
    }
  for (int g = 0; g < ngran; ++g) CHECK(map[g].kind != -1, g);
  for (size_t x = 0; x < kcov.size(); ++x) CHECK(kcov[x] == 1, (long long)x);
  for (size_t x = 0; x < vcov.size(); ++x) CHECK(vcov[x] == 1, (long long)x);

  for (int lane = 0; lane < 64; ++lane) {
    const int half = lane >> 5, l32 = lane & 31;
    // S^T = K Q^T: A row l32 = key 32 kt + l32, k-step s = d-elements [h D/2 + 8 s, +8),
    // which is what the query operand of (l32, h, s) holds.
    for (int kt = 0; kt < 2; ++kt)
      for (int s = 0; s < G::DS; ++s) {
        const uint32_t off = kt * 32 * G::KRB + G::k_rd(l32, half, s);
        CHECK(off % 16 == 0 && off + 16 <= (uint32_t)G::KB, lane, kt, s);
        const Gran& gr = map[off / 16];
        CHECK(gr.kind == 0 && gr.a == 32 * kt + l32 && gr.b == half * (D / 2) + 8 * s, lane, kt, s);
      }
    // O^T += V^T P^T: element t of the B operand pb[jj] is P of register e = 8 jj + t,
    // the key acc_key(kt, e, h) of the stage's half-step kt; element t of the A operand
    // must be v of the same key and of head-dimension row dt 32 + l32.
    for (int kt = 0; kt < 2; ++kt)
      for (int dt = 0; dt < G::DT; ++dt)
        for (int jj = 0; jj < 2; ++jj) {
          const uint32_t off = dt * 32 * G::VRB + G::v_rd(l32, 2 * (2 * kt + jj) + half);
          CHECK(off % 16 == 0 && off >= (uint32_t)G::KB && off + 16 <= (uint32_t)G::SB, lane, kt,
                dt);
          const Gran& gr = map[off / 16];
          CHECK(gr.kind == 1 && gr.a == dt * 32 + l32, lane, kt, dt);
          for (int t = 0; t < 8; ++t) {
            const int key_v = up::attn::swap_bits23(gr.b + t);
            const int key_p = up::attn::acc_key(kt, 8 * jj + t, half);
            CHECK(key_v == key_p, lane, kt, t);
          }
        }
  }
  // The 16 accumulator registers of the two lane halves of a column cover the 32 rows of
  // the tile once, and the output stores cover head-dimension rows dt 32 + [0, 32) once.
  std::vector<int> rows(32, 0), dims(D, 0);
  for (int half = 0; half < 2; ++half)
    for (int e = 0; e < 16; ++e) rows[up::attn::acc_key(0, e, half)]++;
  for (int r = 0; r < 32; ++r) CHECK(rows[r] == 1, r);
  for (int half = 0; half < 2; ++half)
    for (int dt = 0; dt < G::DT; ++dt)
      for (int eg = 0; eg < 4; ++eg)
        for (int m = 0; m < 4; ++m) {
          // register 4 eg + m holds row 8 eg + 4 h + m of tile dt, stored at dv + m
          const int dv = dt * 32 + 8 * eg + 4 * half;
          CHECK(up::attn::acc_key(0, 4 * eg + m, half) + dt * 32 == dv + m, half, dt, eg);
          dims[dv + m]++;
        }
  for (int d = 0; d < D; ++d) CHECK(dims[d] == 1, d);
  for (int t = 0; t < 64; ++t) CHECK(up::attn::swap_bits23(up::attn::swap_bits23(t)) == t, t);
}

// Range [lo, hi) of element offsets one stage's copies reach, relative to the stage base.
template <int D>
void copy_ranges(int64_t Rp, int64_t* klo, int64_t* khi, int64_t* vlo, int64_t* vhi) {
  using G = up::attn::W8<D>;
  *klo = *vlo = INT64_MAX;
  *khi = *vhi = INT64_MIN;
  for (int tid = 0; tid < G::NT; ++tid) {
    for (int q = 0; q < G::KSPT; ++q) {
      const int64_t o = G::k_src(q, tid);
      if (o < *klo) *klo = o;
      if (o + 8 > *khi) *khi = o + 8;
    }
    for (int q = 0; q < G::VSPT; ++q) {
      const int64_t o = G::v_src(q, tid, Rp);
      if (o < *vlo) *vlo = o;
      if (o + 8 > *vhi) *vhi = o + 8;
    }
  }
}

template <int D>
void part2(int Hq, int Hkv, const std::vector<int>& lens) {
  using G = up::attn::W8<D>;
  const int B = (int)lens.size();
  CHECK(Hq % Hkv == 0 && up::attn::w8_serves(D, Hkv), Hq, Hkv);
  const int gsz = Hq / Hkv;
  const int HQ = gsz % 4 == 0 ? 4 : (gsz % 2 == 0 ? 2 : 1);
  const int TT = 4 / HQ;
  const int tok_tile = 64 * TT;
  // The plan's definitions: cu = prefix sums of the lengths, po = of the lengths
  // rounded up to 64, tp = of the workgroup tiles.
  std::vector<int32_t> cu(B + 1, 0), po(B + 1, 0), tp(B + 1, 0);
  for (int i = 0; i < B; ++i) {
    cu[i + 1] = cu[i] + lens[i];
    po[i + 1] = po[i] + (lens[i] + 63) / 64 * 64;
    tp[i + 1] = tp[i] + (lens[i] + tok_tile - 1) / tok_tile;
  }
  const int64_t R = cu[B], Rp = po[B], tiles = tp[B];
  const int gx = Hkv * (gsz / HQ);
  const int64_t nq = (int64_t)Hq * Rp * D, nk = (int64_t)Hkv * Rp * D, nv = nk;
  const int64_t nkn = (int64_t)Hkv * (Rp / 64), nout = R * Hq * D;
  int64_t klo, khi, vlo, vhi;
  copy_ranges<D>(Rp, &klo, &khi, &vlo, &vhi);
  CHECK(klo == 0 && khi == 64LL * D, klo, khi);
  CHECK(vlo == 0 && vhi == (int64_t)(D - 1) * Rp + 64, vlo, vhi);
  std::vector<uint8_t> written((size_t)(R * Hq * (D / 4)), 0);

  std::vector<int> slot_stage(G::NS), last_read(0), ready(0);
  for (int by = 0; by < tiles; ++by)
    for (int bx = 0; bx < gx; ++bx) {
      const up::attn::Wg w =
          up::attn::wg_of(bx, by, Hq, Hkv, HQ, TT, B, cu.data(), po.data(), tp.data());
      CHECK(w.i >= 0 && w.i < B && lens[w.i] > 0, bx, by, w.i);
      CHECK(by >= tp[w.i] && by < tp[w.i + 1], bx, by, w.i);
      CHECK(w.g >= 0 && w.g < Hkv && w.quad >= 0 && w.quad < gsz / HQ, bx, by);
      CHECK(w.nst >= 1 && w.nst <= w.ntile && w.tile0 < w.ntile, bx, by, w.nst);
      CHECK(w.pbase == po[w.i] && w.pbase % 64 == 0, bx, by);
      const int nst = w.nst;
      // every stage lies inside the request's padded rows and inside kr / vt / kn
      CHECK(w.pbase + 64LL * nst <= po[w.i + 1], bx, by, nst);
      for (int st = 0; st < nst; st += (nst > 2 ? nst - 1 : 1)) {
        const int64_t kb = up::attn::k_stage<D>(w, st, Rp), vb = up::attn::v_stage<D>(w, st, Rp);
        CHECK(kb + klo >= 0 && kb + khi <= nk, bx, by, st);
        CHECK(vb + vlo >= 0 && vb + vhi <= nv, bx, by, st);
        const int64_t ki = up::attn::kn_index(w, st, Rp);
        CHECK(ki >= 0 && ki < nkn, bx, by, st);
      }
      // waves
      up::attn::Wv wv[8];
      for (int wave = 0; wave < 8; ++wave) {
        wv[wave] = up::attn::wave_of(w, wave, Hq, Hkv, HQ);
        const up::attn::Wv& v = wv[wave];
        CHECK(v.head >= w.g * gsz && v.head < (w.g + 1) * gsz, bx, by, wave);
        CHECK(v.act == (v.tw < w.ntile), bx, by, wave);
        if (!v.act) continue;
        CHECK(v.tw < nst && v.tw >= w.tile0, bx, by, wave);
        for (int lane = 0; lane < 64; ++lane) {
          const int half = lane >> 5, l32 = lane & 31;
          const int64_t qs = up::attn::q_src<D>(w, v, l32, half, Rp);
          CHECK(qs >= 0 && qs + D / 2 <= nq, bx, by, wave);
          const int qtok = up::attn::query_token(v, l32);
          CHECK(w.pbase + qtok < po[w.i + 1], bx, by, qtok);
          // unmasked keys are exactly [0, qtok]: half-steps before the diagonal stage
          // (hs < 2 tw) hold keys < 64 tw <= qtok; the diagonal stage masks key > qtok
          CHECK(64 * v.tw <= qtok && qtok < 64 * (v.tw + 1), bx, by, qtok);
          if (qtok >= w.L) continue;
          for (int dt = 0; dt < G::DT; ++dt)
            for (int eg = 0; eg < 4; ++eg) {
              const int dv = dt * 32 + 8 * eg + 4 * half;
              const int64_t oi = up::attn::out_index<D>(cu.data(), w, v, l32, Hq, dv);
              CHECK(oi >= 0 && oi + 4 <= nout && oi % 4 == 0, bx, by, oi);
              uint8_t& c = written[(size_t)(oi / 4)];
              CHECK(c == 0, bx, by, oi);
              c = 1;
            }
        }
      }
      // The ring, in the kernel's program order; barriers are the same for every wave
      // (they depend on nst only), so phases are counted per workgroup.
      std::fill(slot_stage.begin(), slot_stage.end(), -1);
      last_read.assign(nst, -1);
      ready.assign(nst, -1);
      int phase = 0;
      std::vector<int> inflight;   // stages issued and not yet waited for, oldest first
      auto issue = [&](int st) {
        const int slot = st % G::NS;
        const int old = slot_stage[slot];
        if (old >= 0) CHECK(last_read[old] < phase, bx, by, st);   // read before the barrier
        slot_stage[slot] = st;
        inflight.push_back(st);
      };
      auto wait_barrier = [&](int n) {
        CHECK(n % G::SPT == 0, n);
        const size_t keep = (size_t)(n / G::SPT);
        CHECK(inflight.size() >= keep, bx, by, n);
        while (inflight.size() > keep) {
          ready[inflight.front()] = phase + 1;   // complete for everyone after the barrier
          inflight.erase(inflight.begin());
        }
        ++phase;
      };
      auto read = [&](int hs) {
        const int st = hs >> 1;
        CHECK(st >= 0 && st < nst, bx, by, hs);
        CHECK(slot_stage[st % G::NS] == st, bx, by, hs);
        CHECK(ready[st] >= 0 && ready[st] <= phase, bx, by, hs);
        if (phase > last_read[st]) last_read[st] = phase;
      };
      issue(0);
      if (nst > 1) issue(1);
      if (nst > 2) issue(2);
      if (nst > 2) wait_barrier(2 * G::SPT);
      else if (nst > 1) wait_barrier(G::SPT);
      else wait_barrier(0);
      for (int wave = 0; wave < 8; ++wave)
        if (wv[wave].act) read(0);
      std::vector<int> pv_count(8, 0), s_count(8, 1);
      auto body = [&](int wave, int hs) {
        const up::attn::Wv& v = wv[wave];
        const int last_hs = 2 * v.tw + 1;
        if (!v.act || hs > last_hs) return;
        if (hs + 1 <= last_hs) {
          read(hs + 1);   // S^T of the next half-step (and its key-norm entry)
          s_count[wave]++;
        }
        read(hs);         // softmax and P V of this half-step
        pv_count[wave]++;
      };
      for (int st = 0; st < nst; ++st) {
        for (int wave = 0; wave < 8; ++wave) body(wave, 2 * st);
        if (st + 1 < nst) {
          if (st + 2 < nst) wait_barrier(G::SPT);
          else wait_barrier(0);
          if (st + 3 < nst) issue(st + 3);
        }
        for (int wave = 0; wave < 8; ++wave) body(wave, 2 * st + 1);
      }
      CHECK(inflight.empty(), bx, by, (long long)inflight.size());
      for (int wave = 0; wave < 8; ++wave)
        if (wv[wave].act) {
          // every half-step up to the diagonal stage's end: one S^T and one P V each
          CHECK(pv_count[wave] == 2 * wv[wave].tw + 2 && s_count[wave] == 2 * wv[wave].tw + 2, bx,
                by, wave);
        }
    }
  for (size_t x = 0; x < written.size(); ++x) CHECK(written[x] == 1, (long long)x);
  std::printf("launch D=%d Hq=%d Hkv=%d B=%d rows=%lld padded=%lld tiles=%lld grid=%dx%lld: ok\n",
              D, Hq, Hkv, B, (long long)R, (long long)Rp, (long long)tiles, gx, (long long)tiles);
}

// Parts 1 and 2 for the 4-wave kernel (W4): 32-key stages of a 32-key K tile and a
// V^T tile of 32 tokens per row; a wave holds one query head's 32-token tile.
template <int D>
void part1_w4() {
  using G = up::attn::W4<D>;
  const int ngran = G::SB / 16;
  std::vector<Gran> map(ngran);
  std::vector<int> kcov(32 * D / 8, 0), vcov(D * 32 / 8, 0);
  for (int q = 0; q < G::KSPT; ++q)
    for (int tid = 0; tid < G::NT; ++tid) {
      const int wave = tid / 64, lane = tid % 64;
      const uint32_t dst = G::k_dst(q, wave) + 16u * lane;
      CHECK(dst % 16 == 0 && dst + 16 <= (uint32_t)G::KB, q, tid, dst);
      const int src = G::k_src(q, tid);
      CHECK(src % 8 == 0 && src >= 0 && src + 8 <= 32 * D, q, tid, src);
      CHECK(map[dst / 16].kind == -1, q, tid, dst);
      map[dst / 16] = Gran{0, src / D, src % D};
      kcov[src / 8]++;
    }
  for (int q = 0; q < G::VSPT; ++q)
    for (int tid = 0; tid < G::NT; ++tid) {
      const int wave = tid / 64, lane = tid % 64;
      const uint32_t dst = G::v_dst(q, wave) + 16u * lane;
      CHECK(dst % 16 == 0 && dst >= (uint32_t)G::KB && dst + 16 <= (uint32_t)G::SB, q, tid, dst);
      const int64_t Rp = 1 << 20;
      const int64_t src = G::v_src(q, tid, Rp);
      const int row = (int)(src / Rp), tok = (int)(src % Rp);
      CHECK(row >= 0 && row < D && tok % 8 == 0 && tok + 8 <= 32, q, tid, src);
      CHECK(map[dst / 16].kind == -1, q, tid, dst);
      map[dst / 16] = Gran{1, row, tok};
      vcov[(row * 32 + tok) / 8]++;
    }
  for (int g = 0; g < ngran; ++g) CHECK(map[g].kind != -1, g);
  for (size_t x = 0; x < kcov.size(); ++x) CHECK(kcov[x] == 1, (long long)x);
  for (size_t x = 0; x < vcov.size(); ++x) CHECK(vcov[x] == 1, (long long)x);
  for (int lane = 0; lane < 64; ++lane) {
    const int half = lane >> 5, l32 = lane & 31;
    // S^T = K Q^T: A row l32 = the stage's key l32; k-step s = d-elements [h D/2 + 8 s, +8)
    for (int s = 0; s < G::DS; ++s) {
      const uint32_t off = G::k_rd(l32, half, s);
      CHECK(off % 16 == 0 && off + 16 <= (uint32_t)G::KB, lane, s);
      const Gran& gr = map[off / 16];
      CHECK(gr.kind == 0 && gr.a == l32 && gr.b == half * (D / 2) + 8 * s, lane, s);
    }
    // O^T += V^T P^T: element t of pb[jj] is P of register 8 jj + t; granule 2 jj + h of
    // V^T row dt 32 + l32 must hold v of the same keys, in the stored token order.
    for (int dt = 0; dt < G::DT; ++dt)
      for (int jj = 0; jj < 2; ++jj) {
        const uint32_t off = dt * 32 * G::VRB + G::v_rd(l32, 2 * jj + half);
        CHECK(off % 16 == 0 && off >= (uint32_t)G::KB && off + 16 <= (uint32_t)G::SB, lane, dt, jj);
        const Gran& gr = map[off / 16];
        CHECK(gr.kind == 1 && gr.a == dt * 32 + l32, lane, dt, jj);
        for (int t = 0; t < 8; ++t) {
          const int key_v = up::attn::swap_bits23(gr.b + t);
          const int key_p = up::attn::acc_key(0, 8 * jj + t, half);
          CHECK(key_v == key_p, lane, dt, t);
        }
      }
  }
}

template <int D>
void part2_w4(int Hq, int Hkv, const std::vector<int>& lens) {
  using G = up::attn::W4<D>;
  const int B = (int)lens.size();
  CHECK(Hq % Hkv == 0 && !up::attn::w8_serves(D, Hkv), Hq, Hkv);
  const int gsz = Hq / Hkv;
  const int HQ = gsz % 4 == 0 ? 4 : (gsz % 2 == 0 ? 2 : 1);
  const int TT = 4 / HQ;
  const int tok_tile = 32 * TT;
  std::vector<int32_t> cu(B + 1, 0), po(B + 1, 0), tp(B + 1, 0);
  for (int i = 0; i < B; ++i) {
    cu[i + 1] = cu[i] + lens[i];
    po[i + 1] = po[i] + (lens[i] + 63) / 64 * 64;
    tp[i + 1] = tp[i] + (lens[i] + tok_tile - 1) / tok_tile;
  }
  const int64_t R = cu[B], Rp = po[B], tiles = tp[B];
  const int gx = Hkv * (gsz / HQ);
  const int64_t nq = (int64_t)Hq * Rp * D, nk = (int64_t)Hkv * Rp * D, nv = nk;
  const int64_t nout = R * Hq * D;
  int64_t klo = INT64_MAX, khi = INT64_MIN, vlo = INT64_MAX, vhi = INT64_MIN;
  for (int tid = 0; tid < G::NT; ++tid) {
    for (int q = 0; q < G::KSPT; ++q) {
      const int64_t o = G::k_src(q, tid);
      klo = std::min(klo, o);
      khi = std::max(khi, o + 8);
    }
    for (int q = 0; q < G::VSPT; ++q) {
      const int64_t o = G::v_src(q, tid, Rp);
      vlo = std::min(vlo, o);
      vhi = std::max(vhi, o + 8);
    }
  }
  CHECK(klo == 0 && khi == 32LL * D, klo, khi);
  CHECK(vlo == 0 && vhi == (int64_t)(D - 1) * Rp + 32, vlo, vhi);
  std::vector<uint8_t> written((size_t)(R * Hq * (D / 4)), 0);
  std::vector<int> slot_stage(G::NS), last_read, ready;
  for (int by = 0; by < tiles; ++by)
    for (int bx = 0; bx < gx; ++bx) {
      const up::attn::Wg w = up::attn::wg_of(bx, by, Hq, Hkv, HQ, TT, B, cu.data(), po.data(),
                                             tp.data(), up::attn::kSlotsAll, nullptr, 5);
      CHECK(w.i >= 0 && w.i < B && lens[w.i] > 0, bx, by, w.i);
      CHECK(by >= tp[w.i] && by < tp[w.i + 1], bx, by, w.i);
      CHECK(w.g >= 0 && w.g < Hkv && w.quad >= 0 && w.quad < gsz / HQ, bx, by);
      CHECK(w.nst >= 1 && w.nst <= w.ntile && w.tile0 < w.ntile, bx, by, w.nst);
      CHECK(w.ntile == (lens[w.i] + 31) / 32, bx, by, w.ntile);
      CHECK(w.pbase == po[w.i] && w.pbase % 64 == 0, bx, by);
      const int nst = w.nst;
      // every 32-key stage lies inside the request's padded rows and inside kr / vt
      CHECK(w.pbase + 32LL * nst <= po[w.i + 1], bx, by, nst);
      for (int st = 0; st < nst; ++st) {
        const int64_t kb = up::attn::k_stage4<D>(w, st, Rp), vb = up::attn::v_stage4<D>(w, st, Rp);
        CHECK(kb + klo >= 0 && kb + khi <= nk, bx, by, st);
        CHECK(vb + vlo >= 0 && vb + vhi <= nv, bx, by, st);
      }
      up::attn::Wv wv[4];
      for (int wave = 0; wave < 4; ++wave) {
        wv[wave] = up::attn::wave4_of(w, wave, Hq, Hkv, HQ);
        const up::attn::Wv& v = wv[wave];
        CHECK(v.head >= w.g * gsz && v.head < (w.g + 1) * gsz, bx, by, wave);
        CHECK(v.act == (v.tw < w.ntile), bx, by, wave);
        if (!v.act) continue;
        CHECK(v.tw < nst && v.tw >= w.tile0, bx, by, wave);
        for (int lane = 0; lane < 64; ++lane) {
          const int half = lane >> 5, l32 = lane & 31;
          const int64_t qs = up::attn::q_src4<D>(w, v, l32, half, Rp);
          CHECK(qs >= 0 && qs + D / 2 <= nq, bx, by, wave);
          const int qtok = up::attn::query_token4(v, l32);
          CHECK(w.pbase + qtok < po[w.i + 1], bx, by, qtok);
          CHECK(32 * v.tw <= qtok && qtok < 32 * (v.tw + 1), bx, by, qtok);
          if (qtok >= w.L) continue;
          for (int dt = 0; dt < G::DT; ++dt)
            for (int eg = 0; eg < 4; ++eg) {
              const int dv = dt * 32 + 8 * eg + 4 * half;
              const int64_t oi = up::attn::out_index4<D>(cu.data(), w, v, l32, Hq, dv);
              CHECK(oi >= 0 && oi + 4 <= nout && oi % 4 == 0, bx, by, oi);
              uint8_t& c = written[(size_t)(oi / 4)];
              CHECK(c == 0, bx, by, oi);
              c = 1;
            }
        }
      }
      // The ring in the kernel's program order (a stage is one 32-key half-step).
      std::fill(slot_stage.begin(), slot_stage.end(), -1);
      last_read.assign(nst, -1);
      ready.assign(nst, -1);
      int phase = 0;
      std::vector<int> inflight;
      auto issue = [&](int st) {
        const int slot = st % G::NS;
        const int old = slot_stage[slot];
        if (old >= 0) CHECK(last_read[old] < phase, bx, by, st);
        slot_stage[slot] = st;
        inflight.push_back(st);
      };
      auto wait_barrier = [&](int n) {
        CHECK(n % G::SPT == 0, n);
        const size_t keep = (size_t)(n / G::SPT);
        CHECK(inflight.size() >= keep, bx, by, n);
        while (inflight.size() > keep) {
          ready[inflight.front()] = phase + 1;
          inflight.erase(inflight.begin());
        }
        ++phase;
      };
      auto read = [&](int st) {
        CHECK(st >= 0 && st < nst, bx, by, st);
        CHECK(slot_stage[st % G::NS] == st, bx, by, st);
        CHECK(ready[st] >= 0 && ready[st] <= phase, bx, by, st);
        if (phase > last_read[st]) last_read[st] = phase;
      };
      // sync_for(st): wait for stage st + 1 (st + 2 may stay in flight), barrier, refill
      // the slot of stage st - 1 with stage st + 3.  (The statistics stores the kernel
      // counts in the same wait are not stages: the wait still drains stage st + 1.)
      auto sync_for = [&](int st) {
        if (st + 1 >= nst) return;
        if (st + 2 < nst) wait_barrier(G::SPT);
        else wait_barrier(0);
        if (st + 3 < nst) issue(st + 3);
      };
      issue(0);
      if (nst > 1) issue(1);
      if (nst > 2) issue(2);
      if (nst > 2) wait_barrier(2 * G::SPT);
      else if (nst > 1) wait_barrier(G::SPT);
      else wait_barrier(0);
      for (int wave = 0; wave < 4; ++wave)
        if (wv[wave].act) read(0);
      std::vector<int> pv_count(4, 0), s_count(4, 1);
      auto body = [&](int wave, int hs) {
        const up::attn::Wv& v = wv[wave];
        if (!v.act || hs > v.tw) return;
        if (hs + 1 <= v.tw) {
          read(hs + 1);
          s_count[wave]++;
        }
        read(hs);
        pv_count[wave]++;
      };
      for (int st = 0; st < nst; st += 2) {
        sync_for(st);
        for (int wave = 0; wave < 4; ++wave) body(wave, st);
        if (st + 1 < nst) {
          sync_for(st + 1);
          for (int wave = 0; wave < 4; ++wave) body(wave, st + 1);
        }
      }
      CHECK(inflight.empty(), bx, by, (long long)inflight.size());
      for (int wave = 0; wave < 4; ++wave)
        if (wv[wave].act)
          CHECK(pv_count[wave] == wv[wave].tw + 1 && s_count[wave] == wv[wave].tw + 1, bx, by,
                wave);
    }
  for (size_t x = 0; x < written.size(); ++x) CHECK(written[x] == 1, (long long)x);
  std::printf("launch (4-wave) D=%d Hq=%d Hkv=%d B=%d rows=%lld padded=%lld tiles=%lld grid=%dx%lld: ok\n",
              D, Hq, Hkv, B, (long long)R, (long long)Rp, (long long)tiles, gx, (long long)tiles);
}

// Part 4 (with n): the two launches of up_rope_attention_scores.  For a workgroup tile
// of tok_tile tokens, the window launch (slot layout kSlotsWindow) and the rest
// (kSlotsRest) together cover every (request, slot) exactly once; the window launch
// takes exactly the slots whose tokens reach the request's last W = min(n, L) rows.
void part4(const std::vector<int>& lens, int n, int tok_tile) {
  const int B = (int)lens.size();
  std::vector<int32_t> tp(B + 1, 0), wp(B + 1, 0);
  for (int i = 0; i < B; ++i) {
    const int L = lens[i];
    const int nt = (L + tok_tile - 1) / tok_tile;
    const int W = L < n ? L : n;
    const int nw = (n > 0 && L > 0) ? nt - (L - W) / tok_tile : 0;
    tp[i + 1] = tp[i] + nt;
    wp[i + 1] = wp[i] + nw;
  }
  const int64_t tiles = tp[B], wtiles = wp[B];
  std::vector<uint8_t> seen((size_t)tiles, 0);
  for (int mode : {up::attn::kSlotsWindow, up::attn::kSlotsRest}) {
    const int64_t slots = mode == up::attn::kSlotsWindow ? wtiles : tiles - wtiles;
    for (int by = 0; by < slots; ++by) {
      int i = -1, j = -1;
      up::attn::slot_of(mode, by, B, tp.data(), wp.data(), i, j);
      CHECK(i >= 0 && i < B, mode, by, i);
      const int nt = tp[i + 1] - tp[i];
      CHECK(j >= 0 && j < nt, mode, by, j);
      const int L = lens[i];
      const int W = L < n ? L : n;
      const int wt = nt - 1 - j;                    // the tile: tokens [wt tok, (wt+1) tok)
      const bool window = (int64_t)(wt + 1) * tok_tile > L - W;
      CHECK(window == (mode == up::attn::kSlotsWindow), mode, by, wt);
      uint8_t& c = seen[(size_t)(tp[i] + j)];
      CHECK(c == 0, mode, by, j);
      c = 1;
    }
  }
  for (size_t x = 0; x < seen.size(); ++x) CHECK(seen[x] == 1, (long long)x);
  std::printf("slot layouts tile=%d B=%d n=%d tiles=%lld window=%lld: ok\n", tok_tile, B, n,
              (long long)tiles, (long long)wtiles);
}

void part3(int Hq, int Hkv, const std::vector<int>& lens, int n, int G, int tile_tokens) {
  const int B = (int)lens.size();
  const int gs = Hq / Hkv;
  CHECK(G >= 32 && G % 32 == 0 && n > 0, G, n);
  // The score plan's layout: per request nb = ceil(L / G), W = min(n, L), pairs
  // [nb][Hq W] from ml_off, rows [W][Hq] from win_off Hq.
  int64_t ml_off = 0, win_off = 0;
  for (int i = 0; i < B; ++i) {
    const int L = lens[i];
    const int W = L < n ? L : n;
    const int nb = (L + G - 1) / G;
    const int64_t terms = (int64_t)Hq * W;
    std::vector<uint8_t> seen((size_t)(nb * terms), 0), rows((size_t)terms, 0);
    for (int head = 0; head < Hq; ++head) {
      const int g = head / gs;
      for (int wr = 0; wr < W; ++wr) {
        const int qtok = L - W + wr;
        const int tw = qtok / tile_tokens;
        const int last = (tw + 1) * (tile_tokens / 32) - 1;   // the wave's last half-step
        const int64_t e = up::attn::win_term(g, gs, W, wr, head);
        CHECK(e >= 0 && e < terms, i, head, wr);
        CHECK(rows[(size_t)e] == 0, i, head, wr);
        rows[(size_t)e] = 1;
        // the wave reaches every key the row may see
        CHECK((int64_t)(last + 1) * 32 > qtok, i, qtok, last);
        for (int hs = 0; hs <= last; ++hs) {
          if (!up::attn::stats_flush(hs, last, G)) continue;
          const int b = up::attn::stats_block(hs, G);
          if (b >= nb) {
            CHECK((int64_t)hs * 32 >= L, i, hs, b);   // only half-steps past the last key
            continue;
          }
          uint8_t& c = seen[(size_t)(b * terms + e)];
          CHECK(c == 0, i, b, e);
          c = 1;
        }
        for (int b = up::attn::stats_tail_first(last, G); b < nb; ++b) {
          CHECK((int64_t)b * G > qtok, i, b, qtok);   // wholly after the row: no key it sees
          uint8_t& c = seen[(size_t)(b * terms + e)];
          CHECK(c == 0, i, b, e);
          c = 1;
        }
        const int64_t lse = (win_off + wr) * Hq + head;
        CHECK(lse >= win_off * Hq && lse < (win_off + W) * Hq, i, wr, head);
      }
    }
    for (size_t x = 0; x < seen.size(); ++x) CHECK(seen[x] == 1, i, (long long)x);
    for (size_t x = 0; x < rows.size(); ++x) CHECK(rows[x] == 1, i, (long long)x);
    ml_off += nb * terms;
    win_off += W;
  }
  std::printf("statistics tile=%d Hq=%d Hkv=%d B=%d n=%d G=%d pairs=%lld: ok\n", tile_tokens, Hq,
              Hkv, B, n, G, (long long)ml_off);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 5 && argc != 7) {
    std::printf("usage: attn_replay D Hq Hkv L0,L1,... [n G]\n");
    return 2;
  }
  const int D = std::atoi(argv[1]), Hq = std::atoi(argv[2]), Hkv = std::atoi(argv[3]);
  std::vector<int> lens;
  std::string s = argv[4];
  size_t p = 0;
  while (p <= s.size()) {
    const size_t q = s.find(',', p);
    lens.push_back(std::atoi(s.substr(p, q == std::string::npos ? std::string::npos : q - p).c_str()));
    if (q == std::string::npos) break;
    p = q + 1;
  }
  if (argc == 7) {
    const int n = std::atoi(argv[5]), G = std::atoi(argv[6]);
    // the 8-wave kernel's 64-token tiles (d = 64, 128) and the 4-wave kernel's 32
    const int tile = up::attn::w8_serves(D, Hkv) ? 64 : 32;
    part3(Hq, Hkv, lens, n, G, tile);
    const int gsz = Hq / Hkv;
    const int HQ = gsz % 4 == 0 ? 4 : (gsz % 2 == 0 ? 2 : 1);
    part4(lens, n, tile * (4 / HQ));
  }
  if (up::attn::w8_serves(D, Hkv)) {
    if (D == 64) {
      part1<64>();
      part2<64>(Hq, Hkv, lens);
    } else {
      part1<128>();
      part2<128>(Hq, Hkv, lens);
    }
  } else if (D == 64) {
    part1_w4<64>();
    part2_w4<64>(Hq, Hkv, lens);
  } else if (D == 128) {
    part1_w4<128>();
    part2_w4<128>(Hq, Hkv, lens);
  } else if (D == 256) {
    part1_w4<256>();
    part2_w4<256>(Hq, Hkv, lens);
  } else {
    std::printf("head dimensions are 64, 128 and 256\n");
    return 2;
  }
  std::printf("ok\n");
  return 0;
}
